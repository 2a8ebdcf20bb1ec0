// Weight packing into MFMA fragment order (eagle3_pack_weights).
//
// The weight-streaming GEMM reads, per MFMA, a 16 x 32 bf16 A fragment whose
// lane l holds row (l % 16), k-slice 8*(l/16)..+8.  In row-major order the 64
// lanes touch 16 rows x 64 bytes; packed, the fragment is one contiguous 1 KB
// block and a wave's loads walk memory sequentially.
#include "common.hpp"
#include "gemm_rows.hpp"
#include "pack.hpp"
#include "target.hpp"

namespace e3 {

__global__ __launch_bounds__(256) void pack_kernel(const bf16* __restrict__ W, int K, int N, RowMap map,
                                                   uint4* __restrict__ out) {
  const size_t nchunks = (size_t)K / 32;
  const size_t total = (size_t)(N / 16) * nchunks * 64;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(e & 63);
    const size_t c = (e >> 6) % nchunks, t = (e >> 6) / nchunks;
    const size_t row = (size_t)map((int)t, lane & 15);
    out[e] = *(const uint4*)(W + row * K + c * 32 + 8 * (lane >> 4));
  }
}

namespace {
struct Mat {
  int n, k, map;
};
void mats_of(const eagle3_dims& dm, Mat m[6]) {
  const int d = dm.d, F = dm.ffn, qd = dm.n_q_heads * dm.head_dim;
  const int nqkv = (dm.n_q_heads + 2 * dm.n_kv_heads) * dm.head_dim;
  m[0] = {d, 3 * d, MAP_PLAIN};           // fc
  m[1] = {nqkv, 2 * d, MAP_PAIR_HEAD};    // qkv
  m[2] = {d, qd, MAP_PLAIN};              // o
  m[3] = {2 * F, d, MAP_PAIR_FFN};        // gate_up
  m[4] = {d, F, MAP_PLAIN};               // down
  m[5] = {dm.vocab, d, MAP_PLAIN};        // lm
}
size_t mat_bytes(const Mat& m) { return (((size_t)m.n * m.k * 2) + 255) & ~(size_t)255; }
}  // namespace

size_t packed_bytes(const eagle3_dims& dm) {
  Mat m[6];
  mats_of(dm, m);
  size_t b = 0;
  for (int i = 0; i < 6; ++i) b += mat_bytes(m[i]);
  return b;
}

hipError_t pack_weights(const eagle3_dims& dm, const eagle3_weights& src, void* dst, eagle3_weights* packed,
                        hipStream_t st) {
  Mat m[6];
  mats_of(dm, m);
  const void* in[6] = {src.fc, src.qkv, src.o, src.gate_up, src.down, src.lm};
  const void* outp[6];
  unsigned char* base = (unsigned char*)dst;
  for (int i = 0; i < 6; ++i) {
    RowMap map{m[i].map, dm.head_dim, dm.ffn};
    const size_t total = (size_t)(m[i].n / 16) * (m[i].k / 32) * 64;
    int blocks = (int)((total + 255) / 256);
    if (blocks > 65535) blocks = 65535;
    pack_kernel<<<blocks, 256, 0, st>>>((const bf16*)in[i], m[i].k, m[i].n, map, (uint4*)base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    outp[i] = base;
    base += mat_bytes(m[i]);
  }
  *packed = src;
  packed->fc = outp[0];
  packed->qkv = outp[1];
  packed->o = outp[2];
  packed->gate_up = outp[3];
  packed->down = outp[4];
  packed->lm = outp[5];
  packed->layout = EAGLE3_LAYOUT_PACKED;
  return hipSuccess;
}

hipError_t pack_matrix(const void* src, int n, int k, void* dst, hipStream_t st) {
  RowMap map{MAP_PLAIN, 0, 0};
  const size_t total = (size_t)(n / 16) * (k / 32) * 64;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 65535) blocks = 65535;
  pack_kernel<<<blocks, 256, 0, st>>>((const bf16*)src, k, n, map, (uint4*)dst);
  return hipGetLastError();
}

// one target layer: qkv [(Hq+2Hkv)hd, d] (RoPE pairs share a tile), o,
// gate_up (gate/up rows share a tile), down
namespace {
void target_mats_of(const eagle3_dims& dm, Mat m[4]) {
  const int d = dm.d, F = dm.ffn, qd = dm.n_q_heads * dm.head_dim;
  const int nqkv = (dm.n_q_heads + 2 * dm.n_kv_heads) * dm.head_dim;
  m[0] = {nqkv, d, MAP_PAIR_HEAD};
  m[1] = {d, qd, MAP_PLAIN};
  m[2] = {2 * F, d, MAP_PAIR_FFN};
  m[3] = {d, F, MAP_PLAIN};
}
}  // namespace

size_t target_layer_packed_bytes(const eagle3_dims& dm) {
  Mat m[4];
  target_mats_of(dm, m);
  size_t b = 0;
  for (int i = 0; i < 4; ++i) b += mat_bytes(m[i]);
  return b;
}

hipError_t pack_target_layer(const eagle3_dims& dm, const eagle3_target_layer& src, void* dst,
                             eagle3_target_layer* packed, hipStream_t st) {
  Mat m[4];
  target_mats_of(dm, m);
  const void* in[4] = {src.qkv, src.o, src.gate_up, src.down};
  const void* outp[4];
  unsigned char* base = (unsigned char*)dst;
  for (int i = 0; i < 4; ++i) {
    RowMap map{m[i].map, dm.head_dim, dm.ffn};
    const size_t total = (size_t)(m[i].n / 16) * (m[i].k / 32) * 64;
    int blocks = (int)((total + 255) / 256);
    if (blocks > 65535) blocks = 65535;
    pack_kernel<<<blocks, 256, 0, st>>>((const bf16*)in[i], m[i].k, m[i].n, map, (uint4*)base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    outp[i] = base;
    base += mat_bytes(m[i]);
  }
  *packed = src;
  packed->qkv = outp[0];
  packed->o = outp[1];
  packed->gate_up = outp[2];
  packed->down = outp[3];
  return hipSuccess;
}

}  // namespace e3
