// Weight-streaming GEMM for few rows: Y[r, n] = sum_k X[r, k] * W[n, k],
// r < R <= 64, with a fused epilogue.
//
// Batch-1 / batch-64 drafting is bound by HBM: every weight byte is read
// once per round and used for R <= 64 rows.  One workgroup owns 16*T
// weight rows ("a tile") and the whole K range; its waves split K into
// 32*U-wide groups (wave w takes groups w, w+WAVES, ...).  Each lane reads
// 16-byte runs of one weight row straight into MFMA A registers
// (v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16)..+8]); the X rows
// are the B operand (column = X row).  Per-wave partial tiles are summed in
// LDS in a fixed order (deterministic), then the epilogue runs on the
// [16T x R] fp32 tile.
//
// Row maps let a tile hold the two halves of a pair in rows m and m+8:
// RoPE partners (i, i+hd/2) of one head, or the gate/up rows of one FFN
// column.  The epilogue then sees both halves in the same workgroup.
#pragma once
#include <type_traits>

#include "common.hpp"

namespace e3 {

enum { MAP_PLAIN = 0, MAP_PAIR_HEAD = 1, MAP_PAIR_FFN = 2 };

struct RowMap {
  int kind, hd, ffn;
  // Weight row of tile-local row m (0..15) of 16-row tile `tile`.
  __device__ __forceinline__ int operator()(int tile, int m) const {
    if (kind == MAP_PLAIN) return tile * 16 + m;
    if (kind == MAP_PAIR_HEAD) {
      const int tph = hd >> 4, h = tile / tph, t = tile - h * tph, half = hd >> 1;
      return h * hd + (m < 8 ? t * 8 + m : half + t * 8 + (m - 8));
    }
    return m < 8 ? tile * 8 + m : ffn + tile * 8 + (m - 8);
  }
};

// Number of 16-row tiles for N outputs under a map.
static inline int rowmap_tiles(int kind, int N) { return kind == MAP_PLAIN ? N / 16 : N / 16; }

union U4 {
  uint4 u;
  bf16x8 v;
};

// ---------------------------------------------------------------------------
// Plan: tiles per workgroup (T), MFMAs per k-group (U), column tiles (NT =
// ceil(R/16)) and the split-K factor S (workgroups per tile).  Small-N
// matrices are split along K so that the grid fills the chip; the consumer
// kernel adds the partial tiles in split order.
struct RowsPlan {
  int nt, t, u, waves, splits, tiles;
};

// k-steps of 32 per chunk of the register-weight kernel for 17..64 rows
// (rows_rx.hpp) when it runs the split-K layer GEMMs: eight (8 KB of
// weights per lane in flight, one X copy and barrier per 256 k) measured
// 1.6 % faster than four on the target's 61-row and 4 x 64-row forwards and
// level on the batch-64 drafter
constexpr int RX_SPLIT_KU = 8;

// Splits for the register-weight kernel: 8, or 16 past 256 k-steps (8B
// drafter, batch 64, cold weights: QKV and O fastest at 8, fusion at 16),
// halved until every split holds whole chunks (the 8B down projection: 8);
// 0 if none does.
static inline int rx_splits(int K) {
  if (K % 32) return 0;
  const int ns = K / 32;
  int s = ns > 256 ? 16 : 8;
  while (s > 1 && (ns % s || (ns / s) % RX_SPLIT_KU)) s >>= 1;
  return s > 1 ? s : 0;
}

static inline RowsPlan plan_rows(int R, int N, int K, bool bf16, bool allow_split = true, bool packed = false) {
  RowsPlan p;
  p.waves = 4;
  p.nt = (R + 15) / 16;
  if (!bf16) {
    p.t = 1;
    p.u = 1;
    p.splits = 1;
    p.tiles = N / 16;
    return p;
  }
  p.t = p.nt == 1 ? 2 : 4;
  p.u = p.nt == 1 ? 4 : 2;
  p.waves = p.nt == 1 ? 8 : 4;
  // up to 16 rows: one 16-row tile per workgroup when two would leave fewer
  // than 192 workgroups (8B O, down and fusion: 256 workgroups)
  if (p.nt == 1 && N / 32 < 192) p.t = 1;
  p.tiles = (N / 16 + p.t - 1) / p.t;
  const int ngroups = K / (32 * p.u);
  int smax = ngroups / p.waves;
  if (smax < 1) smax = 1;
  int s = (1024 + p.tiles - 1) / p.tiles;
  if (s > smax) s = smax;
  // up to 16 rows, at most one workgroup per CU: no split.  The tile streams
  // as fast whole as split (measured on the 8B QKV, O, down and fusion and
  // the 70B O, down and fusion shapes), and the fused epilogue replaces a
  // partial-sum pass.  More tiles than CUs (70B QKV, 320) keep the split.
  if (p.nt == 1 && p.tiles <= 256) s = 1;
  // more than 16 rows: eight splits, halved while a split would hold fewer
  // than 32 k-steps of 32 (measured on the 8B batch-64 shapes: QKV, down and
  // fusion are fastest with eight splits; O streams as fast with four as
  // with eight, and the norm kernel that adds its partials reads half as
  // much; odd counts leave uneven k ranges)
  if (p.nt >= 2) {
    s = 8;
    while (s > 1 && K / 32 / s < 32) s >>= 1;
    // packed weights, up to 64 rows: the register-weight kernel's splits
    if (packed && R <= 64 && rx_splits(K) > 0) s = rx_splits(K);
  }
  if (s < 1 || !allow_split || R > 64) s = 1;
  p.splits = s;
  return p;
}

// fp32 floats of the split-K partials of a plan: [splits][R][N]
static inline size_t rows_partial_floats(const RowsPlan& p, int R, int N) {
  return p.splits > 1 ? (size_t)p.splits * R * N : 0;
}

// Compute a [16*T x R] tile over k in [k0, k1) into LDS `tile_out` (layout
// [16*T][RP], RP = 16*NT), bf16 operands on MFMA.  k-group g (32*U wide)
// feeds U MFMAs; MFMA j covers k in [kb+32j, kb+32j+32) and lane l brings
// the 8 elements at kb + 32j + 8*(l/16) of weight row l%16 (A) and of X row
// l%16 (B): the four lanes of a row read 64 contiguous bytes.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Weight fragment loads bypass reuse-oriented caching (nontemporal): every
// weight byte is read exactly once per launch.
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int T, int NT, int U, int WAVES, bool PACKED>
__device__ __forceinline__ void rows_tile_bf16(const bf16* __restrict__ X, int ldx, int R,
                                               const bf16* __restrict__ W, int ldw, int k0, int k1,
                                               const int* wrows /*[16*T] in LDS*/, int tile0,
                                               int ntiles16, float* red /*[WAVES][T][NT][256]*/,
                                               float* tile_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, q4 = lane >> 4;
  constexpr int KG = 32 * U;
  // row-major: lane reads W[row][k + 8*q4 ..]; packed: fragment (tile, chunk) is
  // a contiguous 1 KB block and lane l reads its 16 bytes at l*16.
  const bf16* wp[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (PACKED) {
      const int t16 = min(tile0 + t, ntiles16 - 1);
      wp[t] = W + ((size_t)t16 * (ldw / 32) * 64 + lane) * 8;
    } else {
      wp[t] = W + (size_t)wrows[t * 16 + m] * ldw + q4 * 8;
    }
  }
  // element offset of k (a multiple of 32) inside a lane's stream
  auto woff = [&](int k) -> size_t { return PACKED ? (size_t)(k / 32) * 64 * 8 : (size_t)k; };
  const bf16* xp[NT];
  bool xv[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    const int r = c * 16 + m;
    xv[c] = r < R;
    xp[c] = X + (size_t)(xv[c] ? r : 0) * ldx + q4 * 8;
  }
  f32x4 acc[T][NT];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ngroups = (k1 - k0) / KG;
  for (int g = wave; g < ngroups; g += WAVES) {
    const int kb = k0 + g * KG;
    U4 a[T][U], b[NT][U];
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
      for (int t = 0; t < T; ++t) a[t][j].u = ld_stream(wp[t] + woff(kb + j * 32));
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if (xv[c]) b[c][j].u = *(const uint4*)(xp[c] + kb + j * 32);
        else b[c][j].u = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int c = 0; c < NT; ++c)
          acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t][j].v, b[c][j].v, acc[t][c], 0, 0, 0);
  }
  // k tail in 32-wide chunks (one MFMA each), spread over the waves.
  const int kdone = k0 + ngroups * KG;
  const int ntail = (k1 - kdone) / 32;
  for (int c32 = wave; c32 < ntail; c32 += WAVES) {
    const int kb = kdone + c32 * 32;
    U4 a[T], b[NT];
#pragma unroll
    for (int t = 0; t < T; ++t) a[t].u = ld_stream(wp[t] + woff(kb));
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      if (xv[c]) b[c].u = *(const uint4*)(xp[c] + kb);
      else b[c].u = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int c = 0; c < NT; ++c)
        acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t].v, b[c].v, acc[t][c], 0, 0, 0);
  }
  // Output layout of the 16x16 MFMA: lane l holds D[4(l/16)+i][l%16].
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(((wave * T + t) * NT + c) << 8) + ((q4 * 4 + i) << 4) + m] = acc[t][c][i];
  __syncthreads();
  constexpr int RP = 16 * NT + 1;  // padded: column reads of a tile row stay conflict-free
  for (int e = threadIdx.x; e < T * NT * 256; e += WAVES * 64) {
    const int t = e / (NT * 256), rem = e - t * NT * 256, c = rem >> 8, mm = (rem >> 4) & 15,
              n = rem & 15;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += red[(((w * T + t) * NT + c) << 8) + (mm << 4) + n];
    tile_out[(t * 16 + mm) * RP + c * 16 + n] = s;
  }
  __syncthreads();
}

// fp32 operands (small fp32 drafters): plain FMA, one output per thread at a
// time, K in order.
template <int T, int NT, int WAVES>
__device__ __forceinline__ void rows_tile_f32(const float* __restrict__ X, int ldx, int R,
                                              const float* __restrict__ W, int ldw, int K,
                                              const int* wrows, float* tile_out) {
  constexpr int RP = 16 * NT + 1;  // padded: column reads of a tile row stay conflict-free
  for (int e = threadIdx.x; e < 16 * T * R; e += WAVES * 64) {
    const int mm = e / R, r = e - mm * R;
    const float* wp = W + (size_t)wrows[mm] * ldw;
    const float* xp = X + (size_t)r * ldx;
    float s = 0.f;
    for (int k = 0; k < K; ++k) s = fmaf(xp[k], wp[k], s);
    tile_out[mm * RP + r] = s;
  }
  __syncthreads();
}

// Epilogues with a `Pre` type do part of their work before the k loop
// (epi.pre(tile16, R) for each of the workgroup's tiles), where its latency
// hides behind the weight stream; the result comes back with the tile.
struct EpiNoPre {
  struct Pre {};
};
template <class E, class = void>
struct RowsPre : std::false_type {};
template <class E>
struct RowsPre<E, std::void_t<typename E::Pre>> : std::true_type {};

// ---------------------------------------------------------------------------
// The kernel: blockIdx.x = tile * splits + split.  With splits > 1 each
// workgroup covers 1/splits of K and its epilogue (EpiPartial) stores the
// partial tile; the consumer kernel adds the partials in split order.
template <typename TW, int T, int NT, int U, int WAVES, bool PACKED, class Epi>
__global__ __launch_bounds__(WAVES * 64) void rows_gemm_kernel(const TW* __restrict__ X, int ldx,
                                                               int R, const TW* __restrict__ W,
                                                               int K, int ntiles16, int splits,
                                                               RowMap map, Epi epi) {
  constexpr int RP = 16 * NT + 1;  // padded: column reads of a tile row stay conflict-free
  constexpr int TILE = 16 * T * RP;
  __shared__ int wrows[16 * T];
  __shared__ float tile[TILE];
  extern __shared__ float red[];
  const int wg_tile = blockIdx.x / splits, split = blockIdx.x - wg_tile * splits;
  for (int i = threadIdx.x; i < 16 * T; i += WAVES * 64) {
    const int t16 = wg_tile * T + i / 16;
    wrows[i] = t16 < ntiles16 ? map(t16, i & 15) : map(0, i & 15);
  }
  __syncthreads();
  using PreT = typename std::conditional<RowsPre<Epi>::value, Epi, EpiNoPre>::type::Pre;
  PreT pre[T];
  if constexpr (RowsPre<Epi>::value) {
#pragma unroll
    for (int t = 0; t < T; ++t) pre[t] = epi.pre(min(wg_tile * T + t, ntiles16 - 1), R);
  }
  if constexpr (sizeof(TW) == 2) {
    constexpr int KG = 32 * U;
    const int ng = K / KG;
    const int g0 = (int)((long)ng * split / splits), g1 = (int)((long)ng * (split + 1) / splits);
    const int k0 = g0 * KG, k1 = split == splits - 1 ? K : g1 * KG;
    rows_tile_bf16<T, NT, U, WAVES, PACKED>((const bf16*)X, ldx, R, (const bf16*)W, K, k0, k1, wrows,
                                            wg_tile * T, ntiles16, red, tile);
  } else {
    rows_tile_f32<T, NT, WAVES>((const float*)X, ldx, R, (const float*)W, K, K, wrows, tile);
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int t16 = wg_tile * T + t;
    if constexpr (RowsPre<Epi>::value) {
      if (t16 < ntiles16) epi(t16, tile + t * 16 * RP, RP, R, split, pre[t]);
    } else {
      if (t16 < ntiles16) epi(t16, tile + t * 16 * RP, RP, R, split);
    }
  }
}

// ---------------------------------------------------------------------------
// Epilogues.  `tile` is [16][RP] fp32 (row m = tile-local weight row, column
// r = X row).  They run with all threads of the block.

// out[r, n] = v  (float or bf16-rounded), n = map(tile, m).
template <typename TO>
struct EpiStore {
  TO* out;
  int ldo;
  RowMap map;
  __device__ void rebase(int r0) { out += (size_t)r0 * ldo; }
  __device__ void operator()(int tile16, const float* tile, int RP, int R, int) const {
    for (int e = threadIdx.x; e < 16 * R; e += blockDim.x) {
      const int r = e >> 4, m = e & 15;  // 16 threads write one output row's 16 columns
      Elem<TO>::st(out, (size_t)r * ldo + map(tile16, m), tile[m * RP + r]);
    }
  }
};

// LM head for the top-k: fp32 logits out[r, n] (plain map) and, per X row
// and 16-column tile, {max, sum of exp(v - max)} over the tile's 16 logits
// (sum 0 for an all -inf tile).  The 16 threads of one row are the 16 lanes
// of a DPP row, so both go through the fixed row16 trees.
//
// The pairs of row r sit at part[r][slot] with slots grouped by XCD:
// workgroups are dealt to the 8 XCDs in turn, so workgroup g (tiles g*tpw..)
// writes slot (g%8)*per_x + (g/8)*tpw + t.  Each cache line of the array is
// then written from one XCD's L2; interleaved 16-byte pieces from all eight
// cost the LM head 8 us per launch (measured, 8B shape).  The slots of the
// tile numbers past the last tile (up to 8*per_x) get {-inf, 0}, written by
// the workgroup of the last tile, so a reader needs no validity test.
struct TileSlots {
  int nt16, tpw, per_x;  // per_x = tpw * ceil(ceil(nt16/tpw) / 8)
  __host__ __device__ int count() const { return 8 * per_x; }
  __device__ __forceinline__ int slot(int tile16) const {
    const int g = tile16 / tpw, t = tile16 - g * tpw;
    return (g & 7) * per_x + (g >> 3) * tpw + t;
  }
  // tile of a slot, or -1 for a slot no workgroup writes
  __device__ __forceinline__ int tile(int s) const {
    const int x = s / per_x, rem = s - x * per_x, q = rem / tpw, t = rem - q * tpw;
    const int t16 = (q * 8 + x) * tpw + t;
    return t16 < nt16 ? t16 : -1;
  }
};
static inline TileSlots tile_slots(int nt16, int tpw) {
  const int nwg = (nt16 + tpw - 1) / tpw;
  return TileSlots{nt16, tpw, tpw * ((nwg + 7) / 8)};
}

struct EpiLogitsTiles {
  float* out;
  int ldo;
  float2* part;  // [R][slots.count()]
  TileSlots slots;
  __device__ void operator()(int tile16, const float* tile, int RP, int R, int) const {
    const int s = slots.slot(tile16);
    for (int e = threadIdx.x; e < 16 * R; e += blockDim.x) {
      const int r = e >> 4, m = e & 15;
      const float v = tile[m * RP + r];
      out[(size_t)r * ldo + tile16 * 16 + m] = v;
      const float mx = row16_max(v);
      const float sm = row16_sum(mx == -INFINITY ? 0.f : expf(v - mx));
      if (m == 0) part[(size_t)r * slots.count() + s] = make_float2(mx, sm);
    }
    if (tile16 == slots.nt16 - 1) {
      const int npad = slots.count() - slots.nt16;
      for (int e = threadIdx.x; e < npad * R; e += blockDim.x) {
        const int i = e / R, r = e - i * R;
        part[(size_t)r * slots.count() + slots.slot(slots.nt16 + i)] = make_float2(-INFINITY, 0.f);
      }
    }
  }
};

// Split-K partial: part[split][r][n] = v with n = map(tile, m) (natural
// output order whatever the tile's row pairing).
struct EpiPartial {
  float* part;
  int N;
  RowMap map;
  size_t sstride = 0;  // floats between splits; 0: R * N (the launch's own rows)
  __device__ void rebase(int r0) { part += (size_t)r0 * N; }
  __device__ size_t split_off(int split, int R) const { return (size_t)split * (sstride ? sstride : (size_t)R * N); }
  __device__ void operator()(int tile16, const float* tile, int RP, int R, int split) const {
    float* out = part + split_off(split, R);
    for (int e = threadIdx.x; e < 16 * R; e += blockDim.x) {
      const int r = e / 16, m = e - r * 16;
      out[(size_t)r * N + map(tile16, m)] = tile[m * RP + r];
    }
  }
  // The kernels of 17..64 rows hand over the whole workgroup tile: a thread
  // task (row r, tile t, half h) stores the 8 consecutive output columns
  // map(t16, 8h) .. +7 as two 16-byte stores, so that a row's columns leave
  // in runs of whole 32-byte sectors instead of 4-byte scatters (the
  // epilogue of the split-K layer GEMMs is about twice as fast, measured).
  // Every map keeps rows 8h..8h+7 of a tile on consecutive columns.
  static constexpr bool kWhole = true;
  __device__ void whole(int wg, const float* tile, int RP, int R, int NB, int ntiles16, float*, int split) const {
    float* out = part + split_off(split, R);
    for (int e = threadIdx.x; e < R * NB * 2; e += blockDim.x) {
      const int r = e / (NB * 2), q = e - r * (NB * 2), t = q >> 1, h = q & 1;
      const int t16 = wg * NB + t;
      if (t16 >= ntiles16) continue;
      const float* src = tile + (t * 16 + h * 8) * RP + r;
      const float4 a = make_float4(src[0], src[RP], src[2 * RP], src[3 * RP]);
      const float4 b = make_float4(src[4 * RP], src[5 * RP], src[6 * RP], src[7 * RP]);
      float4* dst = (float4*)(out + (size_t)r * N + map(t16, h * 8));
      dst[0] = a;
      dst[1] = b;
    }
  }
};

// out[r, n] = res[r, n] + v  (fp32 residual stream).
struct EpiResidual {
  float* out;
  const float* res;
  int ld;
  __device__ void operator()(int tile16, const float* tile, int RP, int R, int) const {
    for (int e = threadIdx.x; e < 16 * R; e += blockDim.x) {
      const int r = e >> 4, m = e & 15;
      const size_t i = (size_t)r * ld + tile16 * 16 + m;
      out[i] = res[i] + tile[m * RP + r];
    }
  }
};

// z[r, c] = silu(gate) * up for the 8 FFN columns c of a MAP_PAIR_FFN tile
// (rows m < 8 gate, m + 8 the matching up row), rounded to TO.
template <typename TO>
struct EpiSwiGLU {
  TO* z;
  int ffn;
  __device__ void rebase(int r0) { z += (size_t)r0 * ffn; }
  __device__ void operator()(int tile16, const float* tile, int RP, int R, int) const {
    for (int e = threadIdx.x; e < 8 * R; e += blockDim.x) {
      const int r = e >> 3, m = e & 7;
      const float g = tile[m * RP + r], u = tile[(m + 8) * RP + r];
      const float s = g / (1.f + expf(-g));
      Elem<TO>::st(z, (size_t)r * ffn + tile16 * 8 + m, s * u);
    }
  }
  // The kernels of 17..64 rows hand over the whole workgroup tile: a thread
  // task (row r, tile t) computes the tile's 8 outputs of row r (the same
  // arithmetic as above) and stores them together, one 16-byte store for
  // bf16 (ffn is a multiple of 32, so every run is aligned).
  static constexpr bool kWhole = true;
  __device__ void whole(int wg, const float* tile, int RP, int R, int NB, int ntiles16, float*, int) const {
    for (int e = threadIdx.x; e < R * NB; e += blockDim.x) {
      const int r = e / NB, t = e - r * NB;
      const int t16 = wg * NB + t;
      if (t16 >= ntiles16) continue;
      const float* c = tile + t * 16 * RP + r;
      float o[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float g = c[m * RP], u = c[(m + 8) * RP];
        const float s = g / (1.f + expf(-g));
        o[m] = s * u;
      }
      TO* dst = z + (size_t)r * ffn + t16 * 8;
      if constexpr (sizeof(TO) == 2) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(o[2 * i]) | ((uint32_t)f2bf(o[2 * i + 1]) << 16);
        *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        ((float4*)dst)[0] = make_float4(o[0], o[1], o[2], o[3]);
        ((float4*)dst)[1] = make_float4(o[4], o[5], o[6], o[7]);
      }
    }
  }
};

// Where the k/v of query row r go (draft step): committed cache row
// ctx_len[b] + rr (COMMIT, contiguous or paged) or tree slot slot_base + rr.
struct KVDest {
  void* k;
  void* v;
  void* tk;
  void* tv;
  const int32_t* ctx_len;
  const int32_t* block_table;
  int cap, max_blocks, block_size, rows, mode, slot_base, hkv, hd;
  int row0;  // global index of the launch's first row
  // Element offset of (row r, kv head g, dim 0); `tree` tells which buffer.
  __device__ __forceinline__ size_t off(int r_local, int g, bool& tree) const {
    const int r = r_local + row0;
    const int b = r / rows, rr = r - b * rows;
    if (mode == EAGLE3_TREE) {
      tree = true;
      return ((size_t)(b * EAGLE3_MAX_TREE_SLOTS + slot_base + rr) * hkv + g) * hd;
    }
    tree = false;
    const int crow = ctx_len[b] + rr;
    if (block_table) {
      const int blk = block_table[(size_t)b * max_blocks + crow / block_size];
      return ((size_t)blk * block_size + crow % block_size) * hkv * hd + (size_t)g * hd;
    }
    return (((size_t)b * cap + crow) * hkv + g) * hd;
  }
};

// QKV epilogue for a MAP_PAIR_HEAD tile: rows m and m+8 are the RoPE pair
// (i, i + hd/2) of one head, i = t*8 + m.  q goes to q_out [R][Hq*hd];
// k/v go to the KV destination.  Values are rounded to TO after RoPE.  The
// rotation's cos/sin (fp64 angle pos * theta^(-2i/hd)) depend only on the
// row's position and i: the rows GEMM computes them before its k loop (Pre,
// thread elements e = tid and tid + blockDim), the skinny kernel inline.
template <typename TO>
struct EpiQKV {
  TO* q_out;
  const int32_t* pos;  // [R]
  KVDest dst;
  int hq;
  float theta;
  struct Pre {
    float c[2], s[2];
  };
  __device__ __forceinline__ void rope(int r, int i, float& c, float& s) const {
    const double inv = pow((double)theta, -(2.0 * i) / (double)dst.hd);
    const double ang = (double)pos[r] * inv;
    double sd, cd;
    sincos(ang, &sd, &cd);
    c = (float)cd;
    s = (float)sd;
  }
  __device__ Pre pre(int tile16, int R) const {
    const int tph = dst.hd >> 4, head = tile16 / tph, t = tile16 - head * tph;
    Pre p;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = threadIdx.x + u * blockDim.x;
      p.c[u] = 1.f;
      p.s[u] = 0.f;
      if (e < 8 * R && head < hq + dst.hkv) rope(e >> 3, t * 8 + (e & 7), p.c[u], p.s[u]);
    }
    return p;
  }
  __device__ void store(int tile16, const float* tile, int RP, int R, int e, float c, float s) const {
    const int hd = dst.hd, tph = hd >> 4, head = tile16 / tph, t = tile16 - head * tph;
    const int half = hd >> 1;
    const int r = e >> 3, m = e & 7;
    const int i = t * 8 + m;  // pair index within the head
    float a = tile[m * RP + r], b = tile[(m + 8) * RP + r];
    if (head < hq + dst.hkv) {  // q or k: rotate
      const float a2 = a * c - b * s, b2 = b * c + a * s;
      a = a2;
      b = b2;
    }
    if (head < hq) {
      const size_t o = (size_t)r * hq * hd + (size_t)head * hd;
      Elem<TO>::st(q_out, o + i, a);
      Elem<TO>::st(q_out, o + i + half, b);
    } else {
      const bool isk = head < hq + dst.hkv;
      const int g = isk ? head - hq : head - hq - dst.hkv;
      bool tree;
      const size_t o = dst.off(r, g, tree);
      TO* base = (TO*)(isk ? (tree ? dst.tk : dst.k) : (tree ? dst.tv : dst.v));
      Elem<TO>::st(base, o + i, a);
      Elem<TO>::st(base, o + i + half, b);
    }
  }
  __device__ void operator()(int tile16, const float* tile, int RP, int R, int, const Pre& p) const {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = threadIdx.x + u * blockDim.x;
      if (e < 8 * R) store(tile16, tile, RP, R, e, p.c[u], p.s[u]);
    }
  }
  __device__ void operator()(int tile16, const float* tile, int RP, int R, int) const {
    const int tph = dst.hd >> 4, head = tile16 / tph, t = tile16 - head * tph;
    for (int e = threadIdx.x; e < 8 * R; e += blockDim.x) {
      float c = 1.f, s = 0.f;
      if (head < hq + dst.hkv) rope(e >> 3, t * 8 + (e & 7), c, s);
      store(tile16, tile, RP, R, e, c, s);
    }
  }
};

}  // namespace e3
