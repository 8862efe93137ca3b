// Host-side check of the expert-GEMM kernel choices: prints, for one layer
// shape and batch, the row tile of each GEMM (and the output columns per
// block of the direct gate/up and the tiled down projection) and how the shared expert's
// GEMMs are launched, as the library's own plan_layer_gemms() decides them
// (the function the staged layer calls).  Links ffn.hip; launches nothing.
#include <cstdio>
#include <cstdlib>

#include "moe_kernels.h"

using namespace moe;

int main(int argc, char** argv) {
  if (argc != 8) {
    std::fprintf(stderr, "usage: tile_choice H I_loc I_shared E E_loc k T\n");
    return 2;
  }
  const int H = std::atoi(argv[1]), I = std::atoi(argv[2]), Is = std::atoi(argv[3]);
  const int E = std::atoi(argv[4]), E_loc = std::atoi(argv[5]), k = std::atoi(argv[6]);
  const int T = std::atoi(argv[7]);
  const GemmPlan p = plan_layer_gemms(1, T, k, E, E_loc, H, I, Is);
  std::printf("gate_up %d down %d down_cols %d gate_up_cols %d", p.BM, p.BM_dn,
              p.dn_cols ? p.dn_cols : 256, p.up_pack ? 8 : 16);
  if (Is > 0) {
    static const char* how[] = {"own", "shared", "shared_switched"};
    std::printf(" shared_expert %d shared_gate_up %s shared_down %s shared_gate_up_tile %d "
                "shared_down_tile %d", p.BMs, how[p.up], how[p.dn], p.BMs_up, p.BMs_dn);
  }
  std::printf("\n");
  return 0;
}
