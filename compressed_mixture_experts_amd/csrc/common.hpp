// Shared device helpers and launcher declarations of the ButterflyMoE HIP
// library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

enum Act { ACT_F32 = 0, ACT_BF16 = 1 };

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round two floats to bf16 (nearest-even; one v_cvt_pk_bf16_f32) and pack.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Paired 2-bit substrate code: one 32-bit word holds 16 consecutive ternary
// weights, weight c < 8 as bit 4c+1 (nonzero) and bit 4c+3 (negative), weight
// 8 + c as bits 4c and 4c+2.  Masking the word, or the word shifted left by
// one, leaves eight fp4 e2m1 nibbles (weight c in nibble c): +1 -> 0x2,
// -1 -> 0xA, 0 -> 0x0, which v_cvt_scalef32_pk_bf16_fp4 turns into exact bf16.
__device__ __forceinline__ uint32_t pair2_to_fp4(uint32_t w, bool upper) {
  return (upper ? (w << 1) : w) & 0xAAAAAAAAu;
}

// Load 8 consecutive activations starting at element `i` of `p` as floats.
template <int ACT>
__device__ __forceinline__ void load8(const void* p, size_t i, float v[8]) {
  if constexpr (ACT == ACT_BF16) {
    uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + i);
    v[0] = bf16lo(u.x); v[1] = bf16hi(u.x);
    v[2] = bf16lo(u.y); v[3] = bf16hi(u.y);
    v[4] = bf16lo(u.z); v[5] = bf16hi(u.z);
    v[6] = bf16lo(u.w); v[7] = bf16hi(u.w);
  } else {
    const float4* q = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
    float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Store 8 consecutive activations (rounded to the activation dtype).
template <int ACT>
__device__ __forceinline__ void store8(void* p, size_t i, const float v[8]) {
  if constexpr (ACT == ACT_BF16) {
    uint4 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    u.z = pack_bf16x2(v[4], v[5]);
    u.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p) + i) = u;
  } else {
    float4* q = reinterpret_cast<float4*>(reinterpret_cast<float*>(p) + i);
    q[0] = make_float4(v[0], v[1], v[2], v[3]);
    q[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <int ACT>
__device__ __forceinline__ float load1(const void* p, size_t i) {
  if constexpr (ACT == ACT_BF16) {
    return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(p)[i]) << 16);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

// ---------------------------------------------------------------- ternary code
// Substrate word layout (one 32-bit word per 16 consecutive columns): column
// 2j+h has its nonzero bit at 16h+j and its sign bit at 16h+8+j.  The pair of
// columns (2j, 2j+1) becomes two bf16 values (+1 = 0x3F80, -1 = 0xBF80) in one
// 32-bit word with a shift, two masks and a 24-bit multiply.
__device__ __forceinline__ uint32_t ternary_pair_bf16(uint32_t w, int j) {
  const uint32_t sign = (w << (7 - j)) & 0x80008000u;
  const uint32_t mag = __umul24((w >> j) & 0x00010001u, 0x3F80u);
  return sign | mag;
}

__device__ __forceinline__ float ternary_value(uint32_t w, int c) {
  const int j = c >> 1, h = c & 1;
  const uint32_t nz = (w >> (16 * h + j)) & 1u;
  const uint32_t sg = (w >> (16 * h + 8 + j)) & 1u;
  return nz ? (sg ? -1.0f : 1.0f) : 0.0f;
}

// ---------------------------------------------------------------- launchers
struct RouteArgs {
  const void* x;            // [T][d]
  const void* w_gate;       // [N][d]
  int32_t* topk_idx;        // [T][k]
  float* topk_gate;         // [T][k]
  int32_t T, d, N, k, renorm;
  // per token tile b (route_tile_tokens(T, d, act) tokens, C = that times k slots):
  int32_t* tile_slots;      // [R] slots b C .. b C + C - 1 ordered by expert, ascending within one
  float* tile_gates;        // [R] their gates, same order
  int32_t* tile_start;      // [G][N] position of expert e's first slot in tile b's list
  // optional (bf16): W_g as MFMA operand fragments (gate_frag_bytes), read in
  // place of w_gate when set
  const void* w_frag;
};

// Work record of one tile of the square-expert kernel: up to `rows` (32, 48
// or TILE_ROWS_MAX) consecutive bucket rows of one expert (e = -1: no tile), with
// the rows' flat slots and gates.  Expert e's tiles are records
// floor(off_e / rows) + e + j, j < ceil(cnt_e / rows) (off_e = slots of lower
// experts); the at most one record between two experts' ranges, and past the
// last, is empty.  That is ceil(R / rows) + N records.
constexpr int TILE_ROWS_MAX = 64;
struct TileRec {
  int32_t e, nr, pad0, pad1;
  int32_t slot[TILE_ROWS_MAX];
  float gate[TILE_ROWS_MAX];
};

struct BucketArgs {
  const int32_t* tile_slots;  // RouteArgs::tile_slots
  const float* tile_gates;    // RouteArgs::tile_gates
  const int32_t* tile_start;  // RouteArgs::tile_start
  int32_t* offsets;         // [N+1]
  int32_t* perm;            // [R] bucket position -> flat slot
  TileRec* rec;             // [n_rec] tile records, or null
  int32_t R, N, C, G;       // slots, experts, slots per token tile, token tiles
  int32_t rec_rows;         // rows per tile record (32, 48 or 64)
  int32_t n_rec;            // ceil(R / rec_rows) + N when rec is set
  uint4* zero;              // cleared by the bucketing workgroups when set
  size_t zero16;            // its 16-byte words
};

// Weight preparation for the expert kernels (once per weight set,
// or per call when no prepared buffer is given).
struct PrepArgs {
  const uint32_t* w_packed; // substrate 0, 2-bit packed, w_words words (16 weights each)
  unsigned char* w_out;     // w_fp4 == 0: one byte per weight (bf16 high byte of +-0.5 / 0);
                            // w_fp4 == 1: paired 2-bit codes, one 32-bit word per 16
                            // consecutive weights (pair2_to_fp4 turns a word into two words
                            // of fp4 e2m1 nibbles)
  int32_t w_words;
  int32_t w_fp4;
  const uint32_t* w_packed1; // substrate 1 (FFN down), always fp4; w_words1 may be 0
  unsigned char* w_out1;
  int32_t w_words1;
  const float* theta;       // [N][L][n/2]
  const float* phi;         // [N][L][n/2]
  unsigned char* fac;       // [N][factor_bytes_per_expert] (matrix-core kernel only)
  int32_t fac_log2n;        // 8 or 9 (0: no factors)
  int32_t n_experts;
};

struct FusedArgs {
  const void* x;            // [T][d] bf16
  void* out;                // per-slot rows [R][d] (or y when k == 1; unused with yatom)
  const float* theta;       // [N][L][d/2]
  const float* phi;         // [N][L][d/2]
  const unsigned char* wb;  // substrate: [d][d] bytes (bf16 high byte of +-0.5 / 0) for the
                            // scalar-rotation kernel, [d][d/2] fp4 e2m1 for the matrix-core one
  const unsigned char* fac; // per-expert rotation block factors (matrix-core path)
  const int32_t* offsets;   // [N+1]
  const int32_t* perm;      // [R]
  const float* gate;        // [R]
  float alpha;              // substrate scale
  int32_t rows, n_experts, top_k;
  const TileRec* rec;       // tile records (matrix-core kernel)
  int32_t tile_rows;        // their rows per tile (fused_tile_rows)
  void* yatom;              // bf16 [T][d], zeroed: rows added into it (k = 2) instead of per-slot rows
};

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2):
// map launch index bid (< nb) to a logical index so that each XCD gets one
// contiguous range of logical indices (neighbouring tiles share its L2).
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// DBG: one angle set for all rows; IN: gather token rows into bucket order, B^T;
// MID: FFN middle; OUT: bucket rows to gated slot rows, B; ROT: bucket rows to
// bucket rows, B or B^T (the training path)
enum BflyMode { BFLY_DBG = 0, BFLY_IN = 1, BFLY_MID = 2, BFLY_OUT = 3, BFLY_ROT = 4 };

struct BflyArgs {
  const void* in;           // source rows
  void* out;                // destination rows
  const float* ang0;        // first rotation's angles  [N][L0][n/2]
  const float* ang1;        // second rotation's angles (MID only)
  const int32_t* offsets;   // [N+1] bucket offsets (bucketed modes)
  const int32_t* perm;      // [R] bucket position -> flat slot
  const float* gate;        // [R] gate per flat slot (OUT)
  int32_t rows;             // R (number of rows)
  int32_t n_experts;
  int32_t top_k;            // IN: token = slot / top_k;  OUT: token when k == 1
  int32_t transpose;        // DBG only
  int32_t gelu;             // MID: apply GELU between the two rotations
  const unsigned char* fac; // prepared block factors of ang0's part (butterfly_split.hip), or null
  const unsigned char* fac1; // high part of the FFN middle: those of ang1
};

// Parts of a wide butterfly run as separate passes (butterfly_split.hip).
enum SplitPart {
  SPLIT_LOW = 0,       // stages 0 .. L-5 (in place)
  SPLIT_LOW_T = 1,     // the same, transposed
  SPLIT_HIGH_IN = 2,   // gather x rows, top 4 stages transposed
  SPLIT_HIGH_MID = 3,  // top 4 stages of ang0, GELU, top 4 of ang1 transposed (in place)
  SPLIT_HIGH_OUT = 4,  // top 4 stages, gate, scatter to slot rows
};

struct GemmArgs {
  const void* a;            // [M][K]
  const uint32_t* w;        // [N][K/16]
  void* z;                  // [M][N]
  float alpha;
  int32_t M, N, K;
};

struct GemmFp4Args {
  const void* a;            // [M][K] bf16
  const unsigned char* w;   // [N][K/4] substrate as paired 2-bit codes (pair2_to_fp4)
  void* z;                  // [M][N] bf16
  float alpha;
  int32_t M, N, K;
  // optional epilogue (N = 4096 or 8192): stages 0..7 of each row's expert
  // rotation (on chunks of 256 columns) applied to Z, rows bucketed by expert
  // (offsets [E+1]), lowfac the rotation's prepared factors for those chunks
  const unsigned char* lowfac;
  const int32_t* offsets;
  int32_t n_experts;
};
bool gemm_fp4_low_epilogue_supported(int N);

struct CombineArgs {
  const void* yp;           // [T*k][d] per-slot gated outputs
  void* y;                  // [T][d]
  int32_t T, d, k;
};

// Tokens per router workgroup for T tokens (the bucketing reads its per-tile lists).
int route_tile_tokens(int T, int d, int act);
hipError_t launch_route(const RouteArgs& a, int act, hipStream_t s);
hipError_t launch_bucket(const BucketArgs& a, hipStream_t s);
hipError_t launch_prep(const PrepArgs& a, hipStream_t s);
// Gate matrix as MFMA operand fragments: for 16-expert block b, contraction
// step st of 32 and lane l (expert 16 b + l % 16, indices 32 st + 8 (l / 16)
// .. +7), 16 bytes at ((b (d / 32) + st) 64 + l) 16; experts past N are zero.
size_t gate_frag_bytes(int N, int d);
bool gate_frag_supported(int d);
hipError_t launch_gate_frag(const void* w_gate, void* out, int N, int d, hipStream_t s);
hipError_t launch_butterfly(const BflyArgs& a, int mode, int act, int log2n, hipStream_t s);
// one angle set for all rows (the test hook of bmoe_debug.h)
hipError_t launch_bfly_dbg(const BflyArgs& a, int act, int log2n, hipStream_t s);
// bucket rows to bucket rows, each expert's B (or B^T when transpose), fp32 stages
hipError_t launch_bfly_rot(const BflyArgs& a, int act, int log2n, bool transpose, hipStream_t s);

// Training-path helpers (train.hip).
hipError_t launch_invert_perm(const int32_t* perm, int32_t* qpos, int R, hipStream_t s);
hipError_t launch_gather_rows(const void* x, const int32_t* perm, void* out, int R, int d, int k, int act,
                              hipStream_t s);
hipError_t launch_token_sum(const void* rows, const int32_t* qpos, const float* gate, const float* base, void* out,
                            bool out_f32, int T, int d, int k, int act, hipStream_t s);
hipError_t launch_transpose_packed(const uint32_t* w, uint32_t* wt, int rows, int cols, hipStream_t s);
hipError_t launch_gelu_fwd(const void* h, void* a, size_t n, int act, hipStream_t s);
hipError_t launch_cast_bf16(const float* in, uint16_t* out, size_t n, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);  // bytes a multiple of 4

// A kernel launched with more than the default 64 KiB of dynamic LDS needs its
// limit raised first.  Done before every such launch (host work of the order
// of a microsecond) instead of remembered, so the library keeps no mutable
// state between calls.
inline hipError_t allow_dynamic_lds(const void* kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
}
hipError_t launch_gemm(const GemmArgs& a, int act, hipStream_t s);
bool bfly_split_supported(int log2n);
// Low-part block factors (matrix-core low part, widths 1024 .. 8192): bytes per
// expert, and the launch that builds them from one butterfly's angles.  The
// low part is stages 0 .. L-5 on chunks of 2^(L-4), or with chunks256 (widths
// 4096 and 8192, for the up product's epilogue) stages 0 .. 7 on chunks of 256.
size_t low_factor_bytes(int log2n, bool chunks256 = false);
hipError_t launch_low_factor_prep(const float* ang, unsigned char* out, int n_experts, int log2n,
                                  bool trans, bool chunks256, hipStream_t s);
// High-part block factors (one 16 x 16 block per column, widths 1024 .. 8192).
size_t high_factor_bytes(int log2n);
hipError_t launch_high_factor_prep(const float* ang, unsigned char* out, int n_experts, int log2n,
                                   bool trans, hipStream_t s);
hipError_t launch_bfly_split(const BflyArgs& a, int part, int log2n, hipStream_t s);
// FFN middle of width 8192 after the up product's epilogue (which applied
// stages 0 .. 7 of ang0): stage 8 and the high part of ang0, GELU, the high
// part of ang1 transposed (in place; fac / fac1 the two high parts' factors).
hipError_t launch_bfly_mid_pair(const BflyArgs& a, hipStream_t s);
// Whole butterfly of width 1024 or 2048 in one pass (butterfly_split.hip):
// input rotation (out_mode false: gather token rows, high^T, low^T, rows in
// bucket order) or output rotation (true: low, high, times the gate, per-slot
// rows); fac = the rotation's low-part factors, fac1 = its high-part factors.
bool bfly_full_supported(int log2n);
hipError_t launch_bfly_full(const BflyArgs& a, bool out_mode, int log2n, hipStream_t s);
bool gemm_fp4_supported(int N, int K);
hipError_t launch_gemm_fp4(const GemmFp4Args& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int act, hipStream_t s);
// Backward of a bucketed butterfly pass (butterfly_bwd.hip): workspace bytes and launch.
size_t bfly_bwd_workspace(int log2n, int n_experts, int rows);
bool sgrad_shape_ok(int M, int N);
size_t router_bwd_workspace(int T, int d, int N);
hipError_t launch_gelu_bwd(const void* h, const void* da, void* dh, size_t n, int act, hipStream_t s);
hipError_t launch_router_bwd(const void* x, const void* wg, const int32_t* idx, const float* dgate, float* dx,
                             float* dwg, void* ws, int T, int d, int N, int k, int renorm, int act, hipStream_t s);
hipError_t launch_combine_bwd(const void* dy, const int32_t* slots, const float* gate, const void* o, void* d_rows,
                              float* d_gate, int R, int k, int d, int act, hipStream_t s);
int sgrad_splits(int M, int N, int R, int* kchunk);
size_t sgrad_workspace(int M, int N, int R);
hipError_t launch_sgrad(const void* dz, const void* u, float alpha, float* out, float* part, int R, int M, int N,
                        hipStream_t s);
hipError_t launch_bfly_bwd(const void* x, const void* dy, void* dx, const float* ang, const int32_t* offsets,
                           float* part, float* dang, int rows, int n_experts, int log2n, int transpose, int act,
                           hipStream_t s);

bool fused_square_supported(int log2n);
bool fused_mfma_supported(int log2n);
size_t factor_bytes_per_expert(int log2n);
// Rows per tile of the matrix-core square-expert kernel for `rows` routed rows
// over n_experts experts on the current device: 32 when the 32-row tiles would
// fill two per CU, else 48 when the 48-row tiles fit one per CU, else 64.
int fused_tile_rows(int rows, int n_experts);
hipError_t launch_fused_mfma(const FusedArgs& a, int log2n, hipStream_t s);
hipError_t launch_fused_square(const FusedArgs& a, int log2n, hipStream_t s);


}  // namespace bmoe
