// Host-side argument fuzzing of the C ABI, built with AddressSanitizer on the
// host pass (no GPU needed).  Every call here either is a pure host query
// (sizes, path choice, strings, the GEMM plan) or carries an argument that
// the host checks reject, so nothing is ever enqueued.  Exit status 0 and a
// final "ok" line mean every check held and the sanitizer found nothing.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "moe.h"
#include "moe_kernels.h"

using namespace moe;

namespace {

uint64_t g_state = 0x9e3779b97f4a7c15ull;
uint32_t next_u32() {            // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545f4914f6cdd1dull) >> 32);
}
int pick(const int* v, int n) { return v[next_u32() % n]; }

int g_fail = 0;
#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      std::fprintf(stderr, "check failed: %s: ", #cond);  \
      std::fprintf(stderr, __VA_ARGS__);                  \
      std::fprintf(stderr, "\n");                         \
      if (++g_fail > 20) std::exit(1);                    \
    }                                                     \
  } while (0)

alignas(16) unsigned char g_buf[4096];   // a host stand-in: only its address is read
void* aligned_ptr() { return g_buf; }
void* misaligned_ptr() { return g_buf + 4; }

const int kEdgeT[] = {-2147483647 - 1, -1, 0, 1, 2, 63, 64, 65, 1000, 8192, 65536,
                      1 << 20, 2097151, 2097152, 2147483647};
const int kEdgeE[] = {-1, 0, 1, 2, 8, 32, 64, 127, 128, 256, 257, 1024, 1025, 65536};
const int kEdgeK[] = {-1, 0, 1, 2, 8, 16, 17, 32, 33, 1000};
const int kEdgeH[] = {-32, 0, 1, 31, 32, 64, 4096, 7168, 65536, 2147483616};
const int kEdgeI[] = {-32, 0, 16, 32, 192, 1536, 2048, 14336, 1 << 24};
const int kEdgeMode[] = {-1, 0, 1, 2, 3, 4};
const int kEdgeDt[] = {-1, 0, 1, 2};

moe_layer_desc random_desc() {
  moe_layer_desc d;
  std::memset(&d, 0, sizeof(d));
  d.H = pick(kEdgeH, sizeof(kEdgeH) / sizeof(int));
  d.E = pick(kEdgeE, sizeof(kEdgeE) / sizeof(int));
  d.k = pick(kEdgeK, sizeof(kEdgeK) / sizeof(int));
  d.I_loc = pick(kEdgeI, sizeof(kEdgeI) / sizeof(int));
  d.I_shared = (next_u32() & 3) ? 0 : pick(kEdgeI, sizeof(kEdgeI) / sizeof(int));
  d.mode = pick(kEdgeMode, sizeof(kEdgeMode) / sizeof(int));
  d.dt = pick(kEdgeDt, sizeof(kEdgeDt) / sizeof(int));
  const int r = next_u32() % 4;
  d.e_begin = r == 0 ? 0 : (int)(next_u32() % 1100) - 10;
  d.e_end = r == 0 ? d.E : d.e_begin + (int)(next_u32() % 300) - 5;
  void* p = (next_u32() % 16) ? aligned_ptr() : ((next_u32() & 1) ? misaligned_ptr() : nullptr);
  d.w_router = p;
  d.w13 = aligned_ptr();
  d.w2 = aligned_ptr();
  d.w13_shared = d.I_shared ? aligned_ptr() : nullptr;
  d.w2_shared = d.I_shared ? aligned_ptr() : nullptr;
  return d;
}

// Half of the cases draw from the accepted ranges only, so the size and plan
// arithmetic runs on many accepted shapes too.
moe_layer_desc random_valid_desc() {
  static const int Hs[] = {32, 64, 2048, 4096, 7168, 65536, 2147483616};
  static const int Es[] = {1, 2, 8, 32, 64, 128, 256, 1000, 1024};
  static const int Is[] = {32, 64, 192, 768, 1536, 2048, 14336, 1 << 24};
  moe_layer_desc d;
  std::memset(&d, 0, sizeof(d));
  d.H = Hs[next_u32() % 7];
  d.E = Es[next_u32() % 9];
  const int kmax = d.E < 32 ? d.E : 32;
  d.k = 1 + (int)(next_u32() % kmax);
  d.I_loc = Is[next_u32() % 8];
  d.I_shared = (next_u32() & 1) ? 0 : Is[next_u32() % 8];
  d.mode = (int)(next_u32() % 4);
  d.dt = (int)(next_u32() & 1);
  d.e_begin = (int)(next_u32() % d.E);
  d.e_end = d.e_begin + 1 + (int)(next_u32() % (d.E - d.e_begin));
  d.w_router = aligned_ptr();
  d.w13 = aligned_ptr();
  d.w2 = aligned_ptr();
  d.w13_shared = d.I_shared ? aligned_ptr() : nullptr;
  d.w2_shared = d.I_shared ? aligned_ptr() : nullptr;
  return d;
}

bool desc_valid(const moe_layer_desc& d) {
  return (d.dt == 0 || d.dt == 1) && d.H > 0 && d.H % 32 == 0 && d.E >= 1 && d.k >= 1 &&
         d.k <= d.E && d.mode >= 0 && d.mode <= 3 && d.E <= 1024 && d.k <= 32 && d.I_loc > 0 &&
         d.I_loc % 32 == 0 && d.e_begin >= 0 && d.e_end <= d.E && d.e_begin < d.e_end &&
         d.I_shared >= 0 && d.I_shared % 32 == 0 && d.w_router == (const void*)g_buf;
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
  CHECK(moe_abi_version() == MOE_ABI_VERSION, "version");
  CHECK(std::strlen(moe_source_sha256()) > 0, "stamp");
  for (int s = -3; s < 10; ++s) CHECK(moe_status_str(s) && moe_status_str(s)[0], "status %d", s);

  long long valid_cases = 0;
  for (int it = 0; it < iters; ++it) {
    const moe_layer_desc d = (it & 1) ? random_valid_desc() : random_desc();
    const int T = pick(kEdgeT, sizeof(kEdgeT) / sizeof(int));
    const bool ok = desc_valid(d);
    const bool t_ok = T >= 0 && ok && (long long)T * d.E <= INT_MAX;

    // size queries: 0 exactly when the desc or T is rejected
    const size_t ws = moe_layer_workspace_size(&d, T);
    CHECK((ws > 0) == t_ok, "layer size %zu for T=%d H=%d E=%d k=%d", ws, T, d.H, d.E, d.k);
    if (t_ok) {
      ++valid_cases;
      CHECK(ws >= (size_t)T * d.E * 4, "size below the logits region");
      const int path = moe_layer_path(&d, T);
      CHECK(path == 0 || path == 1, "path %d", path);
      const int cap = (int)(next_u32() % 5000);
      const size_t wc = moe_layer_capacity_workspace_size(&d, T, cap, 0);
      CHECK(wc == ws, "packed capacity layout differs: %zu vs %zu", wc, ws);
      const size_t wp = moe_layer_capacity_workspace_size(&d, T, cap, 1);
      const long long pad = (long long)(d.e_end - d.e_begin) * cap;
      CHECK((wp > 0) == (pad <= INT_MAX), "padded size %zu", wp);
      // the GEMM plan the staged path would take
      const int E_loc = d.e_end - d.e_begin;
      const GemmPlan g = plan_layer_gemms(d.dt, T, d.k, d.E, E_loc, d.H, d.I_loc, d.I_shared);
      CHECK(g.BM == 16 || g.BM == 32 || g.BM == 64 || g.BM == 128 || g.BM == 256, "BM %d", g.BM);
    } else {
      CHECK(moe_layer_path(&d, T) < 0, "path accepted a rejected call");
    }

    // calls that enqueue work: each carries one argument the host rejects
    alignas(16) moe_debug_out dbg;
    std::memset(&dbg, 0, sizeof(dbg));
    void* wsp = aligned_ptr();
    switch (next_u32() % 6) {
      case 0:
        CHECK(moe_layer(&d, T > 0 ? T : 1, nullptr, aligned_ptr(), wsp, ws, &dbg, nullptr) != MOE_OK,
              "layer without x");
        break;
      case 1:
        CHECK(moe_layer_staged(&d, T > 0 ? T : 1, aligned_ptr(), misaligned_ptr(), wsp, ws,
                               nullptr, nullptr) != MOE_OK, "staged with misaligned y");
        break;
      case 2:
        CHECK(moe_layer_decode(&d, -1, aligned_ptr(), aligned_ptr(), wsp, ws, nullptr, nullptr) !=
                  MOE_OK, "decode T=-1");
        break;
      case 3:
        CHECK(moe_layer_capacity(nullptr, T, 16, next_u32() & 1, aligned_ptr(), aligned_ptr(), wsp,
                                 ws, nullptr, nullptr, nullptr) != MOE_OK, "capacity without desc");
        break;
      case 4:
        CHECK(moe_layer_static(&d, T < 0 ? T : -1, aligned_ptr(), aligned_ptr(), nullptr,
                               nullptr) != MOE_OK, "static T<0");
        break;
      default:
        CHECK(moe_layer_status(misaligned_ptr(), 1 << 20, nullptr) == MOE_ERR_INVALID_ARG,
              "status misaligned");
        CHECK(moe_layer_status(aligned_ptr(), 16, nullptr) == MOE_ERR_INVALID_ARG, "status short");
        break;
    }

    // the step-wise entry points, each rejected before any launch
    const int k = d.k, E = d.E, H = d.H;
    const size_t pws = moe_permute_workspace_size(T, k, E);
    CHECK(pws == 0 || (T >= 0 && k >= 1 && E >= 1), "permute size");
    CHECK(moe_route(aligned_ptr(), aligned_ptr(), d.dt, T, H, E, k, d.mode, nullptr, nullptr,
                    nullptr, (int32_t*)aligned_ptr(), (float*)aligned_ptr(), nullptr) != MOE_OK,
          "route without logits");
    CHECK(moe_permute((const int32_t*)aligned_ptr(), T, k, E, 0, E, nullptr, H, d.dt, nullptr,
                      (int32_t*)aligned_ptr(), nullptr, nullptr, nullptr, wsp, pws, nullptr) !=
              MOE_OK, "permute without counts");
    CHECK(moe_permute_capacity((const int32_t*)aligned_ptr(), T, k, E, 0, E, -1, 1, nullptr, H,
                               d.dt, (int32_t*)aligned_ptr(), (int32_t*)aligned_ptr(), nullptr,
                               nullptr, nullptr, nullptr, wsp, pws, nullptr) != MOE_OK,
          "permute negative capacity");
    const size_t gws = moe_grouped_ffn_workspace_size(T, E, H, d.I_loc, d.dt);
    CHECK(moe_grouped_ffn(nullptr, nullptr, nullptr, (const int32_t*)aligned_ptr(), E, T, H,
                          d.I_loc, aligned_ptr(), aligned_ptr(), d.dt, aligned_ptr(), d.dt, wsp,
                          gws, nullptr) != MOE_OK || T == 0, "grouped ffn without x");
    CHECK(moe_combine(aligned_ptr(), d.dt, nullptr, (const float*)aligned_ptr(), T > 0 ? T : 1, k,
                      H, nullptr, aligned_ptr(), d.dt, nullptr) != MOE_OK, "combine without dst_row");
    const int P = pick(kEdgeK, sizeof(kEdgeK) / sizeof(int));
    const size_t kws = moe_pack_workspace_size(T, k, P);
    CHECK(kws == 0 || (T >= 0 && P >= 1 && P <= 64), "pack size");
    CHECK(moe_pack_by_rank((const int32_t*)aligned_ptr(), nullptr, T, k, E, P, nullptr, H, d.dt,
                           nullptr, (int32_t*)aligned_ptr(), nullptr, nullptr, nullptr, nullptr,
                           nullptr, wsp, kws, nullptr) != MOE_OK, "pack without counts");
    CHECK(moe_unpack_sum(aligned_ptr(), d.dt, nullptr, T > 0 ? T : 1, k, H, aligned_ptr(), d.dt,
                         nullptr) != MOE_OK, "unpack without send_row");
    CHECK(moe_reshard_ep_to_tp_pack(aligned_ptr(), nullptr, E, d.I_loc, H, P, d.dt, nullptr,
                                    nullptr, nullptr) != MOE_OK, "reshard without destination");
  }
  if (g_fail) return 1;
  std::printf("ok %d cases, %lld with an accepted desc and T\n", iters, valid_cases);
  return 0;
}
