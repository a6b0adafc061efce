// Tiled W4A16 GEMM: the dense and grouped launchers and the fp16 instances (the kernel is
// in wq_tile_kernel.h; the bf16 instances are in wq_gemm_tile_bf16.hip).
#include "wq_tile_kernel.h"

namespace wq {

hipError_t launch_tile_f16(const TileArgs& p, bool grouped, bool swiglu, bool zp, int gpc,
                           bool tall, hipStream_t stream) {
  return launch_tile_type<false>(p, grouped, swiglu, zp, gpc, tall, stream);
}

constexpr int kCus = 256;

bool tile_is_tall(int m, int n, int gpc, bool fp8) { return tile_tall(false, m, gpc, fp8, n); }

int tile_max_splits(int m, int n, int k, int gpc, bool fp8, bool swiglu) {
  // only 128-row tiles of 4-bit weights with 128- or 64-row units, no SwiGLU, split K, into
  // ranges of at least two groups, at most 16
  if (swiglu || fp8 || gpc > 2 || !tile_tall(false, m, gpc, fp8, n)) return 1;
  const int most = k / kGroup / 2;
  return most > 16 ? 16 : (most < 1 ? 1 : most);
}

int tile_splits(int m, int n, int k, int gpc, bool fp8, bool swiglu) {
  const int most = tile_max_splits(m, n, k, gpc, fp8, swiglu);
  if (most <= 1) return 1;
  const int tm = tile_rows(true);
  const long tiles = (long)(n / TN) * ((m + tm - 1) / tm);
  // About one work-group per CU; two from K = 8192 once the tiles alone fill half the CUs
  // (a longer K gives each tile more work against the same partials).  The best of splits
  // 1-16 in sweeps on MI355X (us): K=4096: N=4096, M=128/200/300/512/1024 (16-128 tiles) s16
  // 26.0, s8 26.5, s4 32.9, s4 36.5, s2 51.3 against s1 63.6-66.8; N=8192, M=128/256/512 s8
  // 28.3, s4 35.5, s2 53.1; N=14336, M=24/64/128 s4 18.8, 23.3, 34.2 against s1 36.8-63.0,
  // M=256 s2 51.5, M=512 s1 75.3.  K=14336, N=4096: M=128/256/512 s16 34.2, s8 45.9, s4 73.2
  // against s1 197-199, M=1024 s4 125.0, M=2048 s2 223.0 against s1 233.7; K=28672, N=8192,
  // M=128/256 s8 73.8, s4 128.9 against s1 384-386.
  const long target = (long)kCus * (k >= 8192 && 2 * tiles >= kCus ? 2 : 1);
  const int splits = (int)(target / tiles);
  return splits > most ? most : (splits < 1 ? 1 : splits);
}

hipError_t launch_gemm_tile(const uint16_t* a, int lda, int m, const uint32_t* b,
                            const uint16_t* s, const uint32_t* z, uint16_t* c, int n, int k,
                            bool swiglu, int gpc, bool bf16, bool fp8, int splits,
                            float* partials, hipStream_t stream) {
  if (splits < 1 || (splits > 1 && (partials == nullptr || swiglu || fp8 || gpc > 2)))
    return hipErrorInvalidValue;
  TileArgs p{};
  p.a = a;
  p.lda = lda;
  p.m = m;
  p.b = b;
  p.s = s;
  p.z = z;
  p.c = c;
  p.n = n;
  p.k = k;
  p.ldc = swiglu ? n / 2 : n;
  p.splits = splits;
  p.partials = partials;
  const bool tall = tile_tall(false, m, gpc, fp8, n);
  if (splits > 1 && !tall) return hipErrorInvalidValue;  // only 128-row tiles split K
  const int tm = tile_rows(tall);
  p.tiles = (n / TN) * ((m + tm - 1) / tm) * splits;
  hipError_t e;
  if (fp8) {
    if (z != nullptr || gpc != 1) return hipErrorInvalidValue;
    e = launch_tile_fp8(p, false, swiglu, bf16, stream);
  } else {
    e = bf16 ? launch_tile_bf16(p, false, swiglu, z != nullptr, gpc, tall, stream)
             : launch_tile_f16(p, false, swiglu, z != nullptr, gpc, tall, stream);
  }
  if (e != hipSuccess || splits == 1) return e;
  return launch_reduce_splits(partials, c, m, n, splits, bf16, stream);
}

hipError_t launch_grouped_tile(const GroupedProblem& g, hipStream_t stream) {
  TileArgs p{};
  p.a = g.a;
  p.lda = g.k;
  p.m = 0;
  p.c = g.y;
  p.n = g.n;
  p.k = g.k;
  p.b_bank = g.b_bank;
  p.b_stride = g.b_stride;
  p.s_bank = g.s_bank;
  p.s_stride = g.s_stride;
  p.z_bank = g.z_bank;
  p.z_stride = g.z_stride;
  p.ex_ids = g.ex_ids;
  p.ex_off = g.ex_off;
  p.ex_pairs = g.ex_pairs;
  p.pair_tok = g.pair_tok;
  p.topk_w = g.topk_w;
  p.n_expert = g.n_expert;
  p.n_active = g.n_active;
  p.n_pairs = g.n_pairs;
  p.n_tokens = g.n_tokens;
  p.splits = 1;
  // Per XCD: an upper bound on its share of big tiles (at most n_pairs / tm full row tiles
  // plus one partial tile per segment) and of small tiles (one per segment); the kernel
  // derives the exact shares from the CSR, and work-groups without a tile exit at once.
  const bool tall = tile_tall(true, 0, g.gpc, g.fp8, g.n);
  const long ntn = g.n / TN;
  const long big = ((long)g.n_pairs / tile_rows(tall) + g.n_active) * ntn;
  const long small = (long)g.n_active * ntn;
  const long tiles = kXcds * ((big + kXcds - 1) / kXcds + (small + kXcds - 1) / kXcds);
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffffL) return hipErrorInvalidConfiguration;
  p.tiles = (int)tiles;
  p.ldc = g.swiglu ? g.n / 2 : g.n;
  if (g.fp8) {
    if (g.z_bank != nullptr || g.gpc != 1) return hipErrorInvalidValue;
    return launch_tile_fp8(p, true, g.swiglu, g.bf16, stream);
  }
  return g.bf16 ? launch_tile_bf16(p, true, g.swiglu, g.z_bank != nullptr, g.gpc, tall, stream)
                : launch_tile_f16(p, true, g.swiglu, g.z_bank != nullptr, g.gpc, tall, stream);
}

}  // namespace wq
