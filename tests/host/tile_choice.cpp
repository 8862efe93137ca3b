// Host-side check of the expert-GEMM kernel choices: prints, for one layer
// shape and batch, the row tile of each GEMM and how the shared expert's
// GEMMs are launched.  Links the library's ffn.hip; launches nothing.
#include <cstdio>
#include <cstdlib>

#include "moe_kernels.h"

using namespace moe;

static int cdiv(int a, int b) { return (a + b - 1) / b; }

int main(int argc, char** argv) {
  if (argc != 8) {
    std::fprintf(stderr, "usage: tile_choice H I_loc I_shared E E_loc k T\n");
    return 2;
  }
  const int H = std::atoi(argv[1]), I = std::atoi(argv[2]), Is = std::atoi(argv[3]);
  const int E = std::atoi(argv[4]), E_loc = std::atoi(argv[5]), k = std::atoi(argv[6]);
  const int T = std::atoi(argv[7]);
  const int mean = cdiv(T * k, E);
  const int BM = ffn_row_tile(1, mean, H, I, T * k < E_loc ? T * k : E_loc);
  const int BM_dn = ffn_down_row_tile(1, mean, H, I, BM);
  std::printf("gate_up %d down %d", BM, BM_dn);
  if (Is > 0) {
    FfnArgs f{}; f.dt = 1; f.y_dt = 1; f.H = H; f.I_loc = I; f.max_tiles = 1;
    FfnArgs fd = f;
    if (BM_dn != BM) fd.map_bm = BM;
    FfnArgs g{}; g.dt = 1; g.y_dt = 1; g.H = H; g.I_loc = Is; g.M_dense = T;
    const int BMs = ffn_row_tile(1, T, H, Is, 1);
    g.max_tiles = cdiv(T, BMs);
    const bool thin = ffn_gate_up_blocks(g, BMs) < 256;
    auto how = [&](const FfnArgs& r, int BMr, bool gate_up) -> const char* {
      if (ffn_can_share_gemm(r, BMr, g, BMs, gate_up)) return "shared";
      if (!thin) return "own";
      FfnArgs g2 = g;
      g2.max_tiles = cdiv(T, BMr);
      return ffn_can_share_gemm(r, BMr, g2, BMr, gate_up) ? "shared_switched" : "own";
    };
    std::printf(" shared_expert %d shared_gate_up %s shared_down %s", BMs, how(f, BM, true),
                how(fd, BM_dn, false));
  }
  std::printf("\n");
  return 0;
}
