// Host side of the C ABI declared in include/bmoe.h, include/bmoe_trace.h,
// include/bmoe_grad.h and (built with -DBMOE_DEBUG_EXPORTS only)
// include/bmoe_debug.h: argument validation (all before any enqueue),
// workspace planning, and the launch sequence of the forward pass on the
// caller's stream.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "bmoe.h"
#include "bmoe_debug.h"
#include "bmoe_grad.h"
#include "bmoe_trace.h"
#include "bmoe_train.h"
#include "common.hpp"

using namespace bmoe;

namespace {

thread_local std::string g_last_error;

bmoe_status fail(bmoe_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
bmoe_status fail(bmoe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bmoe_status ok() {
  g_last_error.clear();
  return BMOE_OK;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int ilog2(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  const void* p;
  size_t bytes;
};
bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

size_t act_size(int act) { return act == BMOE_BF16 ? 2 : 4; }

constexpr int32_t kMaxTokens = 1 << 24;

// Per-device gfx950 check, cached.
std::atomic<int> g_dev_state[64];

bmoe_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BMOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < 64) {
    const int st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return BMOE_OK;
    if (st == 2) return fail(BMOE_ERR_DEVICE, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(BMOE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) g_dev_state[dev].store(good ? 1 : 2, std::memory_order_relaxed);
  if (!good) return fail(BMOE_ERR_DEVICE, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
  return BMOE_OK;
}

bmoe_status check_layer(const bmoe_layer* L) {
  if (!L) return fail(BMOE_ERR_NULL, "layer is NULL");
  if (!is_pow2(L->d_model) || L->d_model < 64 || L->d_model > 8192)
    return fail(BMOE_ERR_SHAPE, "d_model=%d must be a power of two in [64, 8192]", L->d_model);
  if (L->d_ff != 0 && (!is_pow2(L->d_ff) || L->d_ff < 64 || L->d_ff > 8192))
    return fail(BMOE_ERR_SHAPE, "d_ff=%d must be 0 or a power of two in [64, 8192]", L->d_ff);
  if (L->n_experts < 1 || L->n_experts > 256)
    return fail(BMOE_ERR_SHAPE, "n_experts=%d must be in [1, 256]", L->n_experts);
  const int kmax = L->n_experts < 8 ? L->n_experts : 8;
  if (L->top_k < 1 || L->top_k > kmax)
    return fail(BMOE_ERR_SHAPE, "top_k=%d must be in [1, %d]", L->top_k, kmax);
  if (L->act_dtype != BMOE_F32 && L->act_dtype != BMOE_BF16)
    return fail(BMOE_ERR_DTYPE, "act_dtype=%d is not BMOE_F32 or BMOE_BF16", L->act_dtype);
  if (L->ffn_act != BMOE_ACT_NONE && L->ffn_act != BMOE_ACT_GELU_ERF)
    return fail(BMOE_ERR_DTYPE, "ffn_act=%d is unknown", L->ffn_act);
  if (L->d_ff == 0 && L->ffn_act != BMOE_ACT_NONE)
    return fail(BMOE_ERR_DTYPE, "ffn_act must be BMOE_ACT_NONE for a square layer");
  if (L->renorm_gates != 0 && L->renorm_gates != 1)
    return fail(BMOE_ERR_SHAPE, "renorm_gates=%d must be 0 or 1", L->renorm_gates);
  if (L->reserved != 0) return fail(BMOE_ERR_SHAPE, "reserved field must be 0");
  const int nsub = L->d_ff ? 2 : 1;
  if (!L->w_gate) return fail(BMOE_ERR_NULL, "w_gate is NULL");
  if (!aligned(L->w_gate, 16)) return fail(BMOE_ERR_ALIGN, "w_gate is not 16-byte aligned");
  for (int m = 0; m < nsub; ++m) {
    if (!L->w_base[m]) return fail(BMOE_ERR_NULL, "w_base[%d] is NULL", m);
    if (!L->theta[m]) return fail(BMOE_ERR_NULL, "theta[%d] is NULL", m);
    if (!L->phi[m]) return fail(BMOE_ERR_NULL, "phi[%d] is NULL", m);
    if (!aligned(L->w_base[m], 16)) return fail(BMOE_ERR_ALIGN, "w_base[%d] is not 16-byte aligned", m);
    if (!aligned(L->theta[m], 4) || !aligned(L->phi[m], 4))
      return fail(BMOE_ERR_ALIGN, "angles of substrate %d are not 4-byte aligned", m);
  }
  return BMOE_OK;
}

bmoe_status check_prepared(const bmoe_layer* L, size_t need) {
  if (!L->prepared || need == 0) return BMOE_OK;
  if (!aligned(L->prepared, 256)) return fail(BMOE_ERR_ALIGN, "prepared is not 256-byte aligned");
  if (L->prepared_bytes < need)
    return fail(BMOE_ERR_WORKSPACE, "prepared buffer has %zu bytes, %zu needed", L->prepared_bytes, need);
  return BMOE_OK;
}

// Tokens per router tile (and bucketing's slots per tile / k) for this layer.
int32_t router_tile(int32_t T, const bmoe_layer* L) {
  return route_tile_tokens(T, L->d_model, L->act_dtype == BMOE_BF16 ? ACT_BF16 : ACT_F32);
}

// Workspace layout (offsets in bytes, each 256-byte aligned).
struct Plan {
  size_t offsets, perm, idx, gate, tslots, tgates, tstart, rec, bufU, bufZ, prep, total;
  bool fused, mfma;
  int64_t R;
  int32_t tiles;            // router token tiles
  int32_t n_rec;            // tile records of the square-expert matrix-core kernel (0: none)
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Square bf16 layers of width <= 512 run rotations and substrate product in one kernel.
bool use_fused(const bmoe_layer* L) {
  return L->act_dtype == BMOE_BF16 && L->d_ff == 0 &&
         (fused_square_supported(ilog2(L->d_model)) || fused_mfma_supported(ilog2(L->d_model)));
}
// ... with the rotations as block factors on the matrix cores (widths 256, 512)
bool use_fused_mfma(const bmoe_layer* L) { return use_fused(L) && fused_mfma_supported(ilog2(L->d_model)); }
// Top-2 square layers on the matrix-core expert kernel add their gated rows
// straight into y (zeroed by the bucketing kernel) with packed bf16 atomic
// adds: 0 + a + b rounds the same in either order, so the result is
// deterministic and equals the separate combine's, and no per-slot rows
// round-trip HBM.  Other top-k keep the per-slot rows and the combine.
bool fused_adds_into_y(const bmoe_layer* L) { return use_fused_mfma(L) && L->top_k == 2; }

// Substrate m's product as a GEMM Z = U W_m^T: output columns and contraction length.
void sub_shape(const bmoe_layer* L, int m, int32_t& n_out, int32_t& k_in) {
  const int32_t d = L->d_model, f = L->d_ff;
  n_out = f == 0 ? d : m == 0 ? f : d;
  k_in = f == 0 ? d : m == 0 ? d : f;
}

// bf16 rows of width 2^log2n (1024 .. 8192): each butterfly runs as a low and
// a high part, each part over many rows of one expert per workgroup.
bool use_split(const bmoe_layer* L, int log2n) {
  return L->act_dtype == BMOE_BF16 && bfly_split_supported(log2n);
}

// Prepared-weights buffer, 256-aligned sections: [substrate 0 re-encoded |
// substrate 1 re-encoded (FFN) | rotation factors].  Fused square layers: the
// substrate as bytes (widths 64, 128) or paired 2-bit codes (256, 512) plus
// block factors (256, 512).  Other bf16 layers: each substrate whose product
// the matrix-core GEMM covers, as paired 2-bit codes.  fp32 layers: nothing.
// Low-part block factors of the butterflies of width 4096 / 8192 (bf16 layers):
// input rotation theta (transposed), output rotation phi, FFN phi_up, FFN
// theta_dn (transposed).
enum LowSet { LF_IN = 0, LF_OUT = 1, LF_UP = 2, LF_DN = 3, LF_SETS = 4 };

struct PrepLayout {
  size_t w_off[2], w_len[2], fac_off, fac_len, total;
  size_t lf_off[LF_SETS], lf_len[LF_SETS];  // low-part block factors
  bool lf_c256[LF_SETS];                     // ... for stages 0..7 on chunks of 256 (the up product's epilogue)
  size_t hf_off[LF_SETS], hf_len[LF_SETS];  // high-part block factors (one 16 x 16 block per column)
  size_t gf_off, gf_len;                     // gate matrix as MFMA fragments (last)
  bool fp4[2];
};

// Angles, width and orientation of low-factor set k.
void low_set(const bmoe_layer* L, int k, const float*& ang, int& log2n, bool& trans) {
  const bool ffn = L->d_ff != 0;
  switch (k) {
    case LF_IN: ang = L->theta[0]; log2n = ilog2(L->d_model); trans = true; break;
    case LF_OUT: ang = L->phi[ffn ? 1 : 0]; log2n = ilog2(L->d_model); trans = false; break;
    case LF_UP: ang = L->phi[0]; log2n = ffn ? ilog2(L->d_ff) : 0; trans = false; break;
    default: ang = L->theta[1]; log2n = ffn ? ilog2(L->d_ff) : 0; trans = true; break;
  }
}

// The gate matrix in MFMA fragment order, after everything else (bf16 layers).
void add_gate_frags(const bmoe_layer* L, PrepLayout& q) {
  q.gf_len = gate_frag_bytes(L->n_experts, L->d_model);
  if (!q.gf_len) return;
  q.gf_off = align256(q.total);
  q.total = align256(q.gf_off + q.gf_len);
}

PrepLayout prep_layout(const bmoe_layer* L) {
  PrepLayout q{};
  size_t o = 0;
  if (use_fused(L)) {
    const size_t d = size_t(L->d_model);
    q.fp4[0] = use_fused_mfma(L);
    q.w_len[0] = d * d / (q.fp4[0] ? 4 : 1);
    o = align256(q.w_len[0]);
    q.fac_off = o;
    q.fac_len = q.fp4[0] ? size_t(L->n_experts) * factor_bytes_per_expert(ilog2(L->d_model)) : 0;
    q.total = align256(o + q.fac_len);
    if (L->act_dtype == BMOE_BF16) add_gate_frags(L, q);
    return q;
  }
  if (L->act_dtype != BMOE_BF16) return q;
  for (int m = 0; m < (L->d_ff ? 2 : 1); ++m) {
    int32_t n_out, k_in;
    sub_shape(L, m, n_out, k_in);
    if (!gemm_fp4_supported(n_out, k_in)) continue;
    q.fp4[m] = true;
    q.w_off[m] = o;
    q.w_len[m] = size_t(n_out) * size_t(k_in) / 4;
    o = align256(o + q.w_len[m]);
  }
  q.fac_off = o;
  // FFN layers of width d_ff = 4096 / 8192 with a prepared up substrate: the up
  // product's epilogue applies stages 0..7 of phi_up (one pass fewer)
  const bool up_epi = L->d_ff && q.fp4[0] && gemm_fp4_low_epilogue_supported(L->d_ff);
  for (int k = 0; k < LF_SETS; ++k) {
    const float* ang;
    int ln;
    bool tr;
    low_set(L, k, ang, ln, tr);
    if (!ln || !use_split(L, ln)) continue;
    q.lf_c256[k] = k == LF_UP && up_epi;
    if (low_factor_bytes(ln, q.lf_c256[k])) {
      q.lf_off[k] = o;
      q.lf_len[k] = low_factor_bytes(ln, q.lf_c256[k]) * size_t(L->n_experts);
      o = align256(o + q.lf_len[k]);
    }
    if (high_factor_bytes(ln)) {
      q.hf_off[k] = o;
      q.hf_len[k] = high_factor_bytes(ln) * size_t(L->n_experts);
      o = align256(o + q.hf_len[k]);
    }
  }
  q.total = o;
  add_gate_frags(L, q);
  return q;
}

// The up product's epilogue applies stages 0..7 of phi_up (width 4096: its
// whole low part; 8192: the FFN middle then starts with stage 8).
bool up_low_in_gemm(const bmoe_layer* L, const PrepLayout& q) {
  return L->d_ff && q.lf_len[LF_UP] && q.lf_c256[LF_UP];
}

// Launches of the preparation: the substrate / fused-factor kernel when it has
// work, then one builder per low-factor set.
bool prep_has_sub(const PrepLayout& q) { return q.w_len[0] || q.w_len[1] || q.fac_len; }

// Arguments of the prep kernel that fills `buf` (layout q) for layer L.
PrepArgs prep_args(const bmoe_layer* L, const PrepLayout& q, unsigned char* buf) {
  PrepArgs pa{};
  int32_t n_out, k_in;
  sub_shape(L, 0, n_out, k_in);
  pa.w_packed = L->w_base[0];
  pa.w_out = buf + q.w_off[0];
  pa.w_words = q.w_len[0] ? int32_t(int64_t(n_out) * k_in / 16) : 0;
  pa.w_fp4 = q.fp4[0] ? 1 : 0;
  if (L->d_ff && q.w_len[1]) {
    sub_shape(L, 1, n_out, k_in);
    pa.w_packed1 = L->w_base[1];
    pa.w_out1 = buf + q.w_off[1];
    pa.w_words1 = int32_t(int64_t(n_out) * k_in / 16);
  }
  pa.theta = L->theta[0];
  pa.phi = L->phi[0];
  pa.fac = buf + q.fac_off;
  pa.fac_log2n = q.fac_len ? ilog2(L->d_model) : 0;
  pa.n_experts = L->n_experts;
  return pa;
}

Plan make_plan(const bmoe_layer* L, int32_t T) {
  Plan p{};
  const int64_t R = int64_t(T) * L->top_k;
  const size_t s = act_size(L->act_dtype);
  const int64_t d = L->d_model, f = L->d_ff;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  p.offsets = take(size_t(L->n_experts + 1) * 4);
  p.perm = take(size_t(R) * 4);
  p.idx = take(size_t(R) * 4);
  p.gate = take(size_t(R) * 4);
  p.tiles = T > 0 ? int32_t((int64_t(T) + router_tile(T, L) - 1) / router_tile(T, L)) : 0;
  p.tslots = take(size_t(R) * 4);
  p.tgates = take(size_t(R) * 4);
  p.tstart = take(size_t(p.tiles) * L->n_experts * 4);
  p.fused = use_fused(L);
  p.bufU = take(size_t(R) * d * s);                  // U, then Z_down (FFN) or per-slot Y (square)
  p.bufZ = take(p.fused ? 0 : size_t(R) * (f > d ? f : d) * s);  // Z / H / A, then per-slot Y (FFN)
  p.mfma = use_fused_mfma(L);
  // tile records at the smaller tile height (the most records); the call
  // picks the height when it runs
  p.n_rec = p.mfma && R > 0 ? int32_t((R + 31) / 32 + L->n_experts) : 0;
  p.rec = take(size_t(p.n_rec) * sizeof(TileRec));
  p.prep = L->prepared ? 0 : take(prep_layout(L).total);  // prepared data built per call
  p.total = o;
  p.R = R;
  return p;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

#define BMOE_HIP(call)                                                                 \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) return fail(BMOE_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

bmoe_status validate_call(const bmoe_layer* L, const void* x, int32_t T, void* ws, size_t ws_bytes,
                          Plan& plan) {
  bmoe_status st = check_layer(L);
  if (st != BMOE_OK) return st;
  if (T < 0 || T > kMaxTokens) return fail(BMOE_ERR_SHAPE, "T=%d must be in [0, %d]", T, kMaxTokens);
  st = check_prepared(L, prep_layout(L).total);
  if (st != BMOE_OK) return st;
  plan = make_plan(L, T);
  if (T == 0) return BMOE_OK;
  if (!x) return fail(BMOE_ERR_NULL, "x is NULL");
  if (!ws) return fail(BMOE_ERR_NULL, "workspace is NULL");
  if (!aligned(x, 16)) return fail(BMOE_ERR_ALIGN, "x is not 16-byte aligned");
  if (!aligned(ws, 256)) return fail(BMOE_ERR_ALIGN, "workspace is not 256-byte aligned");
  if (ws_bytes < plan.total)
    return fail(BMOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, plan.total);
  const Range rx{x, size_t(T) * L->d_model * act_size(L->act_dtype)};
  if (overlap(rx, Range{ws, plan.total})) return fail(BMOE_ERR_ALIAS, "x overlaps the workspace");
  return BMOE_OK;
}

// The caller's prepared gate fragments, or none (the router then reads W_g).
const void* gate_frags(const bmoe_layer* L) {
  const PrepLayout q = prep_layout(L);
  return L->prepared && q.gf_len ? static_cast<const unsigned char*>(L->prepared) + q.gf_off : nullptr;
}

bmoe_status run_route(const bmoe_layer* L, const void* x, int32_t T, int32_t* idx, float* gate,
                      void* ws, const Plan& p, hipStream_t s) {
  const int act = L->act_dtype == BMOE_BF16 ? ACT_BF16 : ACT_F32;
  RouteArgs ra{x, L->w_gate, idx, gate, T, L->d_model, L->n_experts, L->top_k, L->renorm_gates,
               at<int32_t>(ws, p.tslots), at<float>(ws, p.tgates), at<int32_t>(ws, p.tstart)};
  ra.w_frag = gate_frags(L);
  BMOE_HIP(launch_route(ra, act, s));
  BucketArgs ba{ra.tile_slots, ra.tile_gates, ra.tile_start, at<int32_t>(ws, p.offsets), at<int32_t>(ws, p.perm),
                nullptr, int32_t(p.R), L->n_experts, router_tile(T, L) * L->top_k, p.tiles, 0, 0};
  BMOE_HIP(launch_bucket(ba, s));
  return BMOE_OK;
}

}  // namespace

extern "C" {

size_t bmoe_packed_words(int32_t rows, int32_t cols) {
  if (rows < 1 || cols < 16 || cols % 16) return 0;
  return size_t(rows) * size_t(cols / 16);
}

bmoe_status bmoe_pack_ternary(const int8_t* w, int32_t rows, int32_t cols, uint32_t* out,
                              size_t out_words) {
  if (!w) return fail(BMOE_ERR_NULL, "w is NULL");
  if (!out) return fail(BMOE_ERR_NULL, "out is NULL");
  const size_t need = bmoe_packed_words(rows, cols);
  if (need == 0) return fail(BMOE_ERR_SHAPE, "rows=%d cols=%d: need rows >= 1 and cols a positive multiple of 16", rows, cols);
  if (out_words < need) return fail(BMOE_ERR_SHAPE, "out has %zu words, %zu needed", out_words, need);
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t wd = 0; wd < cols / 16; ++wd) {
      uint32_t word = 0;
      for (int c = 0; c < 16; ++c) {
        const int64_t i = r * cols + wd * 16 + c;
        const int8_t v = w[i];
        if (v < -1 || v > 1)
          return fail(BMOE_ERR_TERNARY, "w[%lld] = %d (row %lld, column %lld) is not in {-1, 0, 1}",
                      (long long)i, int(v), (long long)r, (long long)(wd * 16 + c));
        const int j = c >> 1, h = c & 1;
        if (v != 0) word |= 1u << (16 * h + j);
        if (v < 0) word |= 1u << (16 * h + 8 + j);
      }
      out[r * (cols / 16) + wd] = word;
    }
  }
  return ok();
}

bmoe_status bmoe_workspace_size(const bmoe_layer* layer, int32_t T, size_t* bytes) {
  if (!bytes) return fail(BMOE_ERR_NULL, "bytes is NULL");
  bmoe_status st = check_layer(layer);
  if (st != BMOE_OK) return st;
  if (T < 0 || T > kMaxTokens) return fail(BMOE_ERR_SHAPE, "T=%d must be in [0, %d]", T, kMaxTokens);
  st = check_prepared(layer, prep_layout(layer).total);
  if (st != BMOE_OK) return st;
  *bytes = make_plan(layer, T).total;
  return ok();
}

size_t bmoe_prepared_bytes(const bmoe_layer* layer) {
  if (check_layer(layer) != BMOE_OK) return 0;
  return prep_layout(layer).total;
}

bmoe_status bmoe_prepare(const bmoe_layer* layer, void* prepared, size_t bytes, hipStream_t stream) {
  bmoe_status st = check_layer(layer);
  if (st != BMOE_OK) return st;
  const PrepLayout q = prep_layout(layer);
  if (q.total == 0) return ok();
  if (!prepared) return fail(BMOE_ERR_NULL, "prepared is NULL");
  if (!aligned(prepared, 256)) return fail(BMOE_ERR_ALIGN, "prepared is not 256-byte aligned");
  if (bytes < q.total) return fail(BMOE_ERR_WORKSPACE, "prepared buffer has %zu bytes, %zu needed", bytes, q.total);
  const Range rp{prepared, q.total};
  for (int m = 0; m < (layer->d_ff ? 2 : 1); ++m) {
    int32_t n_out, k_in;
    sub_shape(layer, m, n_out, k_in);
    if (q.w_len[m] && overlap(rp, Range{layer->w_base[m], size_t(n_out) * k_in / 4}))
      return fail(BMOE_ERR_ALIAS, "prepared buffer overlaps a weight array");
  }
  if (q.fac_len) {
    const int64_t d = layer->d_model;
    const size_t angle_bytes = size_t(layer->n_experts) * ilog2(d) * (d / 2) * 4;
    if (overlap(rp, Range{layer->theta[0], angle_bytes}) || overlap(rp, Range{layer->phi[0], angle_bytes}))
      return fail(BMOE_ERR_ALIAS, "prepared buffer overlaps a weight array");
  }
  for (int k = 0; k < LF_SETS; ++k) {
    const float* ang;
    int ln;
    bool tr;
    low_set(layer, k, ang, ln, tr);
    if ((q.lf_len[k] || q.hf_len[k]) && overlap(rp, Range{ang, size_t(layer->n_experts) * ln * (size_t(1) << (ln - 1)) * 4}))
      return fail(BMOE_ERR_ALIAS, "prepared buffer overlaps a weight array");
  }
  if (q.gf_len && overlap(rp, Range{layer->w_gate, size_t(layer->n_experts) * layer->d_model * 2}))
    return fail(BMOE_ERR_ALIAS, "prepared buffer overlaps a weight array");
  st = check_device();
  if (st != BMOE_OK) return st;
  unsigned char* buf = static_cast<unsigned char*>(prepared);
  if (prep_has_sub(q)) BMOE_HIP(launch_prep(prep_args(layer, q, buf), stream));
  if (q.gf_len) BMOE_HIP(launch_gate_frag(layer->w_gate, buf + q.gf_off, layer->n_experts, layer->d_model, stream));
  for (int k = 0; k < LF_SETS; ++k) {
    const float* ang;
    int ln;
    bool tr;
    low_set(layer, k, ang, ln, tr);
    if (q.lf_len[k])
      BMOE_HIP(launch_low_factor_prep(ang, buf + q.lf_off[k], layer->n_experts, ln, tr, q.lf_c256[k], stream));
    if (q.hf_len[k]) BMOE_HIP(launch_high_factor_prep(ang, buf + q.hf_off[k], layer->n_experts, ln, tr, stream));
  }
  return ok();
}

bmoe_status bmoe_route(const bmoe_layer* layer, const void* x, int32_t T, int32_t* topk_idx,
                       float* topk_gate, int32_t* expert_offsets, int32_t* bucket_slots,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  bmoe_status st = validate_call(layer, x, T, workspace, workspace_bytes, p);
  if (st != BMOE_OK) return st;
  if (T == 0) return ok();
  if (!topk_idx || !topk_gate) return fail(BMOE_ERR_NULL, "topk_idx / topk_gate is NULL");
  const size_t rb = size_t(p.R) * 4;
  const Range ri{topk_idx, rb}, rg{topk_gate, rb}, rw{workspace, p.total};
  const Range ro{expert_offsets, size_t(layer->n_experts + 1) * 4}, rs{bucket_slots, rb};
  if (overlap(ri, rw) || overlap(rg, rw) || overlap(ri, rg) || overlap(ro, rw) || overlap(rs, rw) ||
      overlap(ro, ri) || overlap(ro, rg) || overlap(rs, ri) || overlap(rs, rg) || overlap(ro, rs))
    return fail(BMOE_ERR_ALIAS, "route outputs overlap each other or the workspace");
  if (!aligned(topk_idx, 16) || !aligned(topk_gate, 4))
    return fail(BMOE_ERR_ALIGN, "topk_idx must be 16-byte aligned, topk_gate 4-byte aligned");
  st = check_device();
  if (st != BMOE_OK) return st;
  st = run_route(layer, x, T, topk_idx, topk_gate, workspace, p, stream);
  if (st != BMOE_OK) return st;
  if (expert_offsets)
    BMOE_HIP(hipMemcpyAsync(expert_offsets, at<int32_t>(workspace, p.offsets),
                            size_t(layer->n_experts + 1) * 4, hipMemcpyDeviceToDevice, stream));
  if (bucket_slots)
    BMOE_HIP(hipMemcpyAsync(bucket_slots, at<int32_t>(workspace, p.perm), rb, hipMemcpyDeviceToDevice, stream));
  return ok();
}

// Kernel launches of one forward, in order (marks[i] follows launch i-1): at
// most 2 + 2 LF_SETS preparation launches, route and bucket, and 12 for the
// widest FFN layer.
constexpr int kMaxForwardKernels = 2 + 2 * LF_SETS + 2 + 12;
static int forward_kernel_names(const bmoe_layer* L, const char* (&names)[kMaxForwardKernels]) {
  int n = 0;
  if (!L->prepared) {
    const PrepLayout q = prep_layout(L);
    if (prep_has_sub(q)) names[n++] = "prep";
    for (int k = 0; k < LF_SETS; ++k) {
      if (q.lf_len[k]) names[n++] = "prep_lo";
      if (q.hf_len[k]) names[n++] = "prep_hi";
    }
    if (q.gf_len) names[n++] = "prep_gate";
  }
  names[n++] = "route";
  names[n++] = "bucket";
  if (use_fused(L)) {
    names[n++] = "fused";
    if (L->top_k > 1 && !fused_adds_into_y(L)) names[n++] = "combine";
    return n;
  }
  // widths 4096 / 8192 run the input and output rotations as two passes each
  const bool split_d = use_split(L, ilog2(L->d_model)) && !bfly_full_supported(ilog2(L->d_model));
  if (split_d) {
    names[n++] = "bfly_in_hi";
    names[n++] = "bfly_in_lo";
  } else {
    names[n++] = "bfly_in";
  }
  if (L->d_ff == 0) {
    names[n++] = "gemm";
  } else {
    names[n++] = "gemm_up";
    if (use_split(L, ilog2(L->d_ff))) {
      if (!up_low_in_gemm(L, prep_layout(L))) names[n++] = "bfly_mid_lo";
      names[n++] = "bfly_mid_hi";
      names[n++] = "bfly_mid_lo_t";
    } else {
      names[n++] = "bfly_mid";
    }
    names[n++] = "gemm_down";
  }
  if (split_d) {
    names[n++] = "bfly_out_lo";
    names[n++] = "bfly_out_hi";
  } else {
    names[n++] = "bfly_out";
  }
  if (L->top_k > 1) names[n++] = "combine";
  return n;
}

static bmoe_status forward_impl(const bmoe_layer* layer, const void* x, int32_t T, void* y,
                                int32_t* topk_idx, float* topk_gate, void* workspace,
                                size_t workspace_bytes, hipStream_t stream, hipEvent_t* marks,
                                int32_t n_marks) {
  Plan p;
  bmoe_status st = validate_call(layer, x, T, workspace, workspace_bytes, p);
  if (st != BMOE_OK) return st;
  if (T == 0) return ok();
  if (!y) return fail(BMOE_ERR_NULL, "y is NULL");
  if (!aligned(y, 16)) return fail(BMOE_ERR_ALIGN, "y is not 16-byte aligned");
  const size_t s = act_size(layer->act_dtype);
  const Range ry{y, size_t(T) * layer->d_model * s}, rx{x, size_t(T) * layer->d_model * s};
  const Range rw{workspace, p.total};
  const size_t rb = size_t(p.R) * 4;
  const Range ri{topk_idx, rb}, rg{topk_gate, rb};
  if (overlap(ry, rx)) return fail(BMOE_ERR_ALIAS, "y overlaps x");
  if (overlap(ry, rw)) return fail(BMOE_ERR_ALIAS, "y overlaps the workspace");
  if (overlap(ri, ry) || overlap(rg, ry) || overlap(ri, rw) || overlap(rg, rw) || overlap(ri, rg) ||
      overlap(ri, rx) || overlap(rg, rx))
    return fail(BMOE_ERR_ALIAS, "topk outputs overlap x, y, each other or the workspace");
  if ((topk_idx && !aligned(topk_idx, 16)) || (topk_gate && !aligned(topk_gate, 4)))
    return fail(BMOE_ERR_ALIGN, "topk_idx must be 16-byte aligned, topk_gate 4-byte aligned");
  st = check_device();
  if (st != BMOE_OK) return st;

  int launch = 0;
  auto mark = [&]() -> hipError_t {
    if (marks && launch < n_marks && marks[launch]) return hipEventRecord(marks[launch], stream);
    return hipSuccess;
  };
  BMOE_HIP(mark());
#define BMOE_LAUNCH(call) \
  do {                    \
    BMOE_HIP(call);       \
    ++launch;             \
    BMOE_HIP(mark());     \
  } while (0)

  const int act = layer->act_dtype == BMOE_BF16 ? ACT_BF16 : ACT_F32;
  int32_t* idx = topk_idx ? topk_idx : at<int32_t>(workspace, p.idx);
  float* gate = topk_gate ? topk_gate : at<float>(workspace, p.gate);
  const int32_t R = int32_t(p.R);
  const int32_t N = layer->n_experts, k = layer->top_k, d = layer->d_model, f = layer->d_ff;
  int32_t* offsets = at<int32_t>(workspace, p.offsets);
  int32_t* perm = at<int32_t>(workspace, p.perm);
  void* bufU = at<char>(workspace, p.bufU);
  void* bufZ = at<char>(workspace, p.bufZ);
  const int Ld = ilog2(d);

  // prepared weights: given, or built here
  const PrepLayout q = prep_layout(layer);
  const bool fused = p.fused;
  const unsigned char* pbase = static_cast<const unsigned char*>(layer->prepared);
  if (q.total && !pbase) {
    unsigned char* buf = at<unsigned char>(workspace, p.prep);
    if (prep_has_sub(q)) BMOE_LAUNCH(launch_prep(prep_args(layer, q, buf), stream));
    for (int k = 0; k < LF_SETS; ++k) {
      const float* ang;
      int ln;
      bool tr;
      low_set(layer, k, ang, ln, tr);
      if (q.lf_len[k]) BMOE_LAUNCH(launch_low_factor_prep(ang, buf + q.lf_off[k], N, ln, tr, q.lf_c256[k], stream));
      if (q.hf_len[k]) BMOE_LAUNCH(launch_high_factor_prep(ang, buf + q.hf_off[k], N, ln, tr, stream));
    }
    if (q.gf_len) BMOE_LAUNCH(launch_gate_frag(layer->w_gate, buf + q.gf_off, N, d, stream));
    pbase = buf;
  }
  auto lowfac = [&](int k) -> const unsigned char* { return q.lf_len[k] ? pbase + q.lf_off[k] : nullptr; };
  auto highfac = [&](int k) -> const unsigned char* { return q.hf_len[k] ? pbase + q.hf_off[k] : nullptr; };
  const unsigned char* wbytes = q.w_len[0] ? pbase + q.w_off[0] : nullptr;
  const unsigned char* wbytes1 = q.w_len[1] ? pbase + q.w_off[1] : nullptr;
  const unsigned char* fac = q.fac_len ? pbase + q.fac_off : nullptr;
  // substrate product: matrix-core GEMM on a prepared substrate, else the 2-bit LDS-decoding one
  auto substrate_gemm = [&](int m, const void* a_in, void* z_out, int32_t n_out, int32_t k_in) -> hipError_t {
    const unsigned char* wq = m == 0 ? wbytes : wbytes1;
    if (wq) return launch_gemm_fp4(GemmFp4Args{a_in, wq, z_out, layer->w_scale[m], R, n_out, k_in}, stream);
    return launch_gemm(GemmArgs{a_in, layer->w_base[m], z_out, layer->w_scale[m], R, n_out, k_in}, act, stream);
  };
  // router and bucketing
  RouteArgs ra{x, layer->w_gate, idx, gate, T, d, N, k, layer->renorm_gates,
               at<int32_t>(workspace, p.tslots), at<float>(workspace, p.tgates), at<int32_t>(workspace, p.tstart)};
  ra.w_frag = q.gf_len ? pbase + q.gf_off : nullptr;
  BMOE_LAUNCH(launch_route(ra, act, stream));
  TileRec* rec = p.n_rec ? at<TileRec>(workspace, p.rec) : nullptr;
  const int rec_rows = rec ? fused_tile_rows(R, N) : 0;
  BucketArgs ba{ra.tile_slots, ra.tile_gates, ra.tile_start, offsets, perm, rec, R, N,
                router_tile(T, layer) * k, p.tiles, rec_rows,
                rec ? int32_t((R + rec_rows - 1) / rec_rows + N) : 0};
  const bool yatom = fused && fused_adds_into_y(layer);
  if (yatom) {
    ba.zero = reinterpret_cast<uint4*>(y);
    ba.zero16 = size_t(T) * d * 2 / 16;
  }
  BMOE_LAUNCH(launch_bucket(ba, stream));
  if (fused) {
    void* yslot_f = k == 1 ? y : at<char>(workspace, p.bufU);
    FusedArgs fa{x, yslot_f, layer->theta[0], layer->phi[0], wbytes, fac, offsets, perm, gate,
                 layer->w_scale[0], R, N, k, rec, rec_rows};
    if (yatom) fa.yatom = y;
    if (p.mfma) {
      BMOE_LAUNCH(launch_fused_mfma(fa, ilog2(d), stream));
    } else {
      BMOE_LAUNCH(launch_fused_square(fa, ilog2(d), stream));
    }
    if (k > 1 && !yatom) {
      CombineArgs c{yslot_f, y, T, d, k};
      BMOE_LAUNCH(launch_combine(c, act, stream));
    }
    return ok();
  }
  // input rotation: U[q] = B(theta_e)^T x_t
  const bool split_d = use_split(layer, Ld);
  BflyArgs bi{x, bufU, layer->theta[0], nullptr, offsets, perm, nullptr, R, N, k, 0, 0, highfac(LF_IN)};
  if (split_d && bfly_full_supported(Ld)) {
    BflyArgs bf{x, bufU, layer->theta[0], nullptr, offsets, perm, nullptr, R, N, k, 0, 0, lowfac(LF_IN),
                highfac(LF_IN)};
    BMOE_LAUNCH(launch_bfly_full(bf, false, Ld, stream));
  } else if (split_d) {
    BMOE_LAUNCH(launch_bfly_split(bi, SPLIT_HIGH_IN, Ld, stream));
    BflyArgs bl{bufU, bufU, layer->theta[0], nullptr, offsets, perm, nullptr, R, N, k, 0, 0, lowfac(LF_IN)};
    BMOE_LAUNCH(launch_bfly_split(bl, SPLIT_LOW_T, Ld, stream));
  } else {
    BMOE_LAUNCH(launch_butterfly(bi, BFLY_IN, act, Ld, stream));
  }
  void* yslot = nullptr;  // per-slot outputs (k > 1)
  void* zlast = nullptr;
  const float* phi_last = nullptr;
  if (f == 0) {
    BMOE_LAUNCH(substrate_gemm(0, bufU, bufZ, d, d));
    zlast = bufZ;
    yslot = bufU;
    phi_last = layer->phi[0];
  } else {
    const bool up_low = up_low_in_gemm(layer, q);
    if (up_low)
      BMOE_LAUNCH(launch_gemm_fp4(GemmFp4Args{bufU, wbytes, bufZ, layer->w_scale[0], R, f, d, lowfac(LF_UP), offsets, N},
                                  stream));
    else
      BMOE_LAUNCH(substrate_gemm(0, bufU, bufZ, f, d));
    const int gelu = layer->ffn_act == BMOE_ACT_GELU_ERF ? 1 : 0;
    BflyArgs bm{bufZ, bufZ, layer->phi[0], layer->theta[1], offsets, perm, nullptr, R, N, k, 0, gelu,
                highfac(LF_UP), highfac(LF_DN)};
    if (use_split(layer, ilog2(f))) {
      // B(theta_dn)^T GELU(B(phi_up) h) = low^T(theta) high^T(theta) GELU high(phi) low(phi) h
      BflyArgs b1{bufZ, bufZ, layer->phi[0], nullptr, offsets, perm, nullptr, R, N, k, 0, 0, lowfac(LF_UP)};
      if (!up_low) BMOE_LAUNCH(launch_bfly_split(b1, SPLIT_LOW, ilog2(f), stream));
      if (up_low && ilog2(f) == 13) BMOE_LAUNCH(launch_bfly_mid_pair(bm, stream));  // stage 8 first
      else BMOE_LAUNCH(launch_bfly_split(bm, SPLIT_HIGH_MID, ilog2(f), stream));
      BflyArgs b3{bufZ, bufZ, layer->theta[1], nullptr, offsets, perm, nullptr, R, N, k, 0, 0, lowfac(LF_DN)};
      BMOE_LAUNCH(launch_bfly_split(b3, SPLIT_LOW_T, ilog2(f), stream));
    } else {
      BMOE_LAUNCH(launch_butterfly(bm, BFLY_MID, act, ilog2(f), stream));
    }
    BMOE_LAUNCH(substrate_gemm(1, bufZ, bufU, d, f));
    zlast = bufU;
    yslot = bufZ;
    phi_last = layer->phi[1];
  }
  // output rotation, gate, per-slot rows (or y directly when k == 1)
  BflyArgs bo{zlast, k == 1 ? y : yslot, phi_last, nullptr, offsets, perm, gate, R, N, k, 0, 0, highfac(LF_OUT)};
  if (split_d && bfly_full_supported(Ld)) {
    BflyArgs bf{zlast, k == 1 ? y : yslot, phi_last, nullptr, offsets, perm, gate, R, N, k, 0, 0, lowfac(LF_OUT),
                highfac(LF_OUT)};
    BMOE_LAUNCH(launch_bfly_full(bf, true, Ld, stream));
  } else if (split_d) {
    BflyArgs bl{zlast, zlast, phi_last, nullptr, offsets, perm, nullptr, R, N, k, 0, 0, lowfac(LF_OUT)};
    BMOE_LAUNCH(launch_bfly_split(bl, SPLIT_LOW, Ld, stream));
    BMOE_LAUNCH(launch_bfly_split(bo, SPLIT_HIGH_OUT, Ld, stream));
  } else {
    BMOE_LAUNCH(launch_butterfly(bo, BFLY_OUT, act, Ld, stream));
  }
  if (k > 1) {
    CombineArgs c{yslot, y, T, d, k};
    BMOE_LAUNCH(launch_combine(c, act, stream));
  }
#undef BMOE_LAUNCH
  return ok();
}

bmoe_status bmoe_forward(const bmoe_layer* layer, const void* x, int32_t T, void* y,
                         int32_t* topk_idx, float* topk_gate, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return forward_impl(layer, x, T, y, topk_idx, topk_gate, workspace, workspace_bytes, stream,
                      nullptr, 0);
}

// ---- allocation-free forward -------------------------------------------
// The workspace of bmoe_forward_noalloc: a fixed array in device memory, one
// copy per GPU the library runs on, alive until the process ends.  Host code
// never uses the array's name as an address: each device's copy is looked up
// once with hipGetSymbolAddress and that pointer is what the kernels get.
static __device__ __align__(256) unsigned char scratch[BMOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
// per-device address of `scratch` (set on the device's first call; the one
// piece of state the library keeps besides the error string)
std::atomic<void*> g_scratch_ptr[kMaxDevices];

bmoe_status scratch_for_current_device(void** out) {
  int dev = -1;
  BMOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(BMOE_ERR_DEVICE, "device %d is beyond the %d this build serves", dev, kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    BMOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || !aligned(p, 256)) return fail(BMOE_ERR_HIP, "scratch of device %d has no usable address", dev);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return BMOE_OK;
}
}  // namespace

bmoe_status bmoe_forward_noalloc(const bmoe_layer* layer, const void* x, int32_t T, void* y,
                                 int32_t* topk_idx, float* topk_gate, hipStream_t stream) {
  size_t need = 0;
  bmoe_status st = bmoe_workspace_size(layer, T, &need);
  if (st != BMOE_OK) return st;
  if (need > BMOE_NOALLOC_SCRATCH_BYTES)
    return fail(BMOE_ERR_WORKSPACE,
                "this layer at T=%d needs %zu bytes of workspace; the allocation-free forward has a fixed "
                "scratch of %zu bytes (use bmoe_forward with a caller workspace, or fewer tokens per call)",
                T, need, size_t(BMOE_NOALLOC_SCRATCH_BYTES));
  if (T == 0) return ok();
  st = check_device();
  if (st != BMOE_OK) return st;
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != BMOE_OK) return st;
  return forward_impl(layer, x, T, y, topk_idx, topk_gate, ws, BMOE_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0);
}

bmoe_status bmoe_forward_kernels(const bmoe_layer* layer, int32_t* n_kernels, char* names,
                                     size_t names_len) {
  bmoe_status st = check_layer(layer);
  if (st != BMOE_OK) return st;
  if (!n_kernels) return fail(BMOE_ERR_NULL, "n_kernels is NULL");
  const char* nm[kMaxForwardKernels];
  const int n = forward_kernel_names(layer, nm);
  *n_kernels = n;
  if (names && names_len) {
    std::string all;
    for (int i = 0; i < n; ++i) {
      if (i) all += ",";
      all += nm[i];
    }
    std::snprintf(names, names_len, "%s", all.c_str());
  }
  return ok();
}

bmoe_status bmoe_forward_marked(const bmoe_layer* layer, const void* x, int32_t T, void* y,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                                    hipEvent_t* marks, int32_t n_marks) {
  if (n_marks < 0) return fail(BMOE_ERR_SHAPE, "n_marks is negative");
  return forward_impl(layer, x, T, y, nullptr, nullptr, workspace, workspace_bytes, stream, marks,
                      n_marks);
}

static bmoe_status check_bwd_shape(int32_t log2n, int32_t n_experts, int32_t rows) {
  if (log2n < 1 || log2n > 13) return fail(BMOE_ERR_SHAPE, "log2n=%d must be in [1, 13]", log2n);
  if (n_experts < 1 || n_experts > 256) return fail(BMOE_ERR_SHAPE, "n_experts=%d must be in [1, 256]", n_experts);
  if (rows < 0 || int64_t(rows) << log2n > (int64_t(1) << 31) - 1)
    return fail(BMOE_ERR_SHAPE, "rows=%d: must be >= 0 with rows * 2^log2n below 2^31", rows);
  return BMOE_OK;
}

bmoe_status bmoe_butterfly_backward_workspace(int32_t log2n, int32_t n_experts, int32_t rows, size_t* bytes) {
  if (!bytes) return fail(BMOE_ERR_NULL, "bytes is NULL");
  const bmoe_status st = check_bwd_shape(log2n, n_experts, rows);
  if (st != BMOE_OK) return st;
  *bytes = bfly_bwd_workspace(log2n, n_experts, rows);
  return ok();
}

bmoe_status bmoe_butterfly_backward(int32_t log2n, int32_t n_experts, int32_t rows, const int32_t* offsets,
                                    const float* angles, int32_t transpose, int32_t dtype, const void* x,
                                    const void* dy, void* dx, float* dangles, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  bmoe_status st = check_bwd_shape(log2n, n_experts, rows);
  if (st != BMOE_OK) return st;
  if (transpose != 0 && transpose != 1) return fail(BMOE_ERR_SHAPE, "transpose must be 0 or 1");
  if (dtype != BMOE_F32 && dtype != BMOE_BF16) return fail(BMOE_ERR_DTYPE, "dtype=%d is unknown", dtype);
  if (!offsets || !angles || !dangles) return fail(BMOE_ERR_NULL, "offsets / angles / dangles is NULL");
  const size_t need = bfly_bwd_workspace(log2n, n_experts, rows);
  if (rows > 0 && (!x || !dy || !dx)) return fail(BMOE_ERR_NULL, "x / dy / dx is NULL");
  if (need > 0 && !workspace) return fail(BMOE_ERR_NULL, "workspace is NULL");
  const size_t es = dtype == BMOE_BF16 ? 2 : 4;
  if (!aligned(offsets, 4) || !aligned(angles, 4) || !aligned(dangles, 4))
    return fail(BMOE_ERR_ALIGN, "offsets, angles and dangles must be 4-byte aligned");
  const size_t ra = log2n >= 3 ? 16 : es;  // rows of 8 or more elements move in 16-byte vectors
  if (rows > 0 && (!aligned(x, ra) || !aligned(dy, ra) || !aligned(dx, ra)))
    return fail(BMOE_ERR_ALIGN, "x, dy and dx must be %zu-byte aligned", ra);
  if (need > 0 && !aligned(workspace, 16)) return fail(BMOE_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(BMOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  const size_t ab = size_t(n_experts) * log2n * (size_t(1) << (log2n - 1)) * 4;
  const size_t rb = (size_t(rows) << log2n) * es;
  const Range rx{x, rb}, rdy{dy, rb}, rdx{dx, rb}, rda{dangles, ab}, ran{angles, ab},
      rof{offsets, size_t(n_experts + 1) * 4}, rws{workspace, need};
  if (rows > 0 && ((dx != x && overlap(rdx, rx)) || (dx != dy && overlap(rdx, rdy)) || overlap(rdx, ran) ||
                   overlap(rdx, rof) || overlap(rdx, rws) || overlap(rdx, rda)))
    return fail(BMOE_ERR_ALIAS, "dx overlaps an input, the workspace or dangles");
  if (overlap(rda, ran) || overlap(rda, rof) || overlap(rda, rws) || (rows > 0 && (overlap(rda, rx) || overlap(rda, rdy))))
    return fail(BMOE_ERR_ALIAS, "dangles overlaps an input or the workspace");
  if (need > 0 && (overlap(rws, ran) || overlap(rws, rof) || (rows > 0 && (overlap(rws, rx) || overlap(rws, rdy)))))
    return fail(BMOE_ERR_ALIAS, "the workspace overlaps an input");
  st = check_device();
  if (st != BMOE_OK) return st;
  BMOE_HIP(launch_bfly_bwd(x, dy, dx, angles, offsets, static_cast<float*>(workspace), dangles, rows, n_experts,
                           log2n, transpose, dtype == BMOE_BF16 ? ACT_BF16 : ACT_F32, stream));
  return ok();
}

#ifdef BMOE_DEBUG_EXPORTS
bmoe_status bmoe_dbg_butterfly(int32_t log2n, int32_t rows, const float* angles, int32_t transpose,
                               int32_t dtype, const void* in, void* out, hipStream_t stream) {
  if (log2n < 3 || log2n > 13) return fail(BMOE_ERR_SHAPE, "log2n=%d must be in [3, 13]", log2n);
  if (rows < 0) return fail(BMOE_ERR_SHAPE, "rows=%d is negative", rows);
  if (transpose != 0 && transpose != 1) return fail(BMOE_ERR_SHAPE, "transpose must be 0 or 1");
  if (dtype != BMOE_F32 && dtype != BMOE_BF16) return fail(BMOE_ERR_DTYPE, "dtype=%d is unknown", dtype);
  if (rows == 0) return ok();
  if (!angles || !in || !out) return fail(BMOE_ERR_NULL, "angles / in / out is NULL");
  if (!aligned(in, 16) || !aligned(out, 16) || !aligned(angles, 4))
    return fail(BMOE_ERR_ALIGN, "in/out must be 16-byte aligned, angles 4-byte aligned");
  const size_t bytes = size_t(rows) << log2n;
  const size_t s = dtype == BMOE_BF16 ? 2 : 4;
  if (in != out && overlap(Range{in, bytes * s}, Range{out, bytes * s}))
    return fail(BMOE_ERR_ALIAS, "in and out overlap without being the same buffer");
  bmoe_status st = check_device();
  if (st != BMOE_OK) return st;
  BflyArgs a{in, out, angles, nullptr, nullptr, nullptr, nullptr, rows, 1, 1, transpose, 0};
  BMOE_HIP(launch_bfly_dbg(a, dtype == BMOE_BF16 ? ACT_BF16 : ACT_F32, log2n, stream));
  return ok();
}

bmoe_status bmoe_dbg_ternary_gemm(int32_t M, int32_t N, int32_t K, int32_t dtype, const void* a,
                                  const uint32_t* w_packed, float alpha, void* z, hipStream_t stream) {
  if (dtype != BMOE_F32 && dtype != BMOE_BF16) return fail(BMOE_ERR_DTYPE, "dtype=%d is unknown", dtype);
  const int q = dtype == BMOE_BF16 ? 64 : 16;
  if (M < 0 || N < q || K < q || N % q || K % q)
    return fail(BMOE_ERR_SHAPE, "M=%d N=%d K=%d: N and K must be positive multiples of %d", M, N, K, q);
  if (M == 0) return ok();
  if (!a || !w_packed || !z) return fail(BMOE_ERR_NULL, "a / w_packed / z is NULL");
  if (!aligned(a, 16) || !aligned(w_packed, 16) || !aligned(z, 16))
    return fail(BMOE_ERR_ALIGN, "a, w_packed and z must be 16-byte aligned");
  const size_t s = dtype == BMOE_BF16 ? 2 : 4;
  if (overlap(Range{a, size_t(M) * K * s}, Range{z, size_t(M) * N * s}))
    return fail(BMOE_ERR_ALIAS, "z overlaps a");
  bmoe_status st = check_device();
  if (st != BMOE_OK) return st;
  GemmArgs g{a, w_packed, z, alpha, M, N, K};
  BMOE_HIP(launch_gemm(g, dtype == BMOE_BF16 ? ACT_BF16 : ACT_F32, stream));
  return ok();
}

bmoe_status bmoe_dbg_ternary_gemm_fp4(int32_t M, int32_t N, int32_t K, const void* a,
                                      const uint32_t* w_packed, void* w_fp4, float alpha, void* z,
                                      hipStream_t stream) {
  if (M < 0 || N <= 0 || K <= 0 || !gemm_fp4_supported(N, K))
    return fail(BMOE_ERR_SHAPE, "M=%d N=%d K=%d: N must be a positive multiple of 256, K of 128", M, N, K);
  if (M == 0) return ok();
  if (!a || !w_packed || !w_fp4 || !z) return fail(BMOE_ERR_NULL, "a / w_packed / w_fp4 / z is NULL");
  if (!aligned(a, 16) || !aligned(w_packed, 16) || !aligned(w_fp4, 16) || !aligned(z, 16))
    return fail(BMOE_ERR_ALIGN, "a, w_packed, w_fp4 and z must be 16-byte aligned");
  const Range ra{a, size_t(M) * K * 2}, rz{z, size_t(M) * N * 2}, rq{w_fp4, size_t(N) * K / 4},
      rw{w_packed, size_t(N) * K / 4};
  if (overlap(ra, rz) || overlap(rq, ra) || overlap(rq, rz) || overlap(rq, rw))
    return fail(BMOE_ERR_ALIAS, "z / w_fp4 overlap an operand");
  bmoe_status st = check_device();
  if (st != BMOE_OK) return st;
  PrepArgs pa{};
  pa.w_packed = w_packed;
  pa.w_out = static_cast<unsigned char*>(w_fp4);
  pa.w_words = int32_t(int64_t(N) * K / 16);
  pa.w_fp4 = 1;
  BMOE_HIP(launch_prep(pa, stream));
  GemmFp4Args g{a, static_cast<const unsigned char*>(w_fp4), z, alpha, M, N, K};
  BMOE_HIP(launch_gemm_fp4(g, stream));
  return ok();
}

#endif  // BMOE_DEBUG_EXPORTS

const char* bmoe_status_string(bmoe_status s) {
  switch (s) {
    case BMOE_OK: return "BMOE_OK";
    case BMOE_ERR_NULL: return "BMOE_ERR_NULL: a required pointer is NULL";
    case BMOE_ERR_SHAPE: return "BMOE_ERR_SHAPE: a size is outside the supported limits";
    case BMOE_ERR_DTYPE: return "BMOE_ERR_DTYPE: unknown dtype or activation";
    case BMOE_ERR_ALIGN: return "BMOE_ERR_ALIGN: a pointer is misaligned";
    case BMOE_ERR_ALIAS: return "BMOE_ERR_ALIAS: an output overlaps an input or the workspace";
    case BMOE_ERR_WORKSPACE: return "BMOE_ERR_WORKSPACE: workspace too small";
    case BMOE_ERR_TERNARY: return "BMOE_ERR_TERNARY: a substrate value is not in {-1, 0, 1}";
    case BMOE_ERR_HIP: return "BMOE_ERR_HIP: a HIP call or kernel launch failed";
    case BMOE_ERR_DEVICE: return "BMOE_ERR_DEVICE: the current device is not gfx950";
  }
  return "unknown bmoe_status";
}

const char* bmoe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

// ---------------------------------------------------------------- substrate weight gradient
static bmoe_status check_sgrad_shape(int32_t d_out, int32_t d_in, int32_t rows) {
  if (d_out < 128 || d_out > 16384 || d_in < 128 || d_in > 16384 || !sgrad_shape_ok(d_out, d_in))
    return fail(BMOE_ERR_SHAPE, "d_out=%d, d_in=%d: each must be a multiple of 128 in [128, 16384]", d_out, d_in);
  const int32_t d = d_out > d_in ? d_out : d_in;
  if (rows < 0 || int64_t(rows) * d > (int64_t(1) << 31) - 1)
    return fail(BMOE_ERR_SHAPE, "rows=%d: must be >= 0 with rows * max(d_out, d_in) below 2^31", rows);
  return BMOE_OK;
}

bmoe_status bmoe_substrate_grad_workspace(int32_t d_out, int32_t d_in, int32_t rows, size_t* bytes) {
  if (!bytes) return fail(BMOE_ERR_NULL, "bytes is NULL");
  const bmoe_status st = check_sgrad_shape(d_out, d_in, rows);
  if (st != BMOE_OK) return st;
  *bytes = sgrad_workspace(d_out, d_in, rows);
  return ok();
}

bmoe_status bmoe_substrate_grad(int32_t d_out, int32_t d_in, int32_t rows, int32_t dtype, const void* dz,
                                const void* u, float alpha, float* dw, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  bmoe_status st = check_sgrad_shape(d_out, d_in, rows);
  if (st != BMOE_OK) return st;
  if (dtype != BMOE_BF16)
    return fail(BMOE_ERR_DTYPE, "dtype=%d: the substrate gradient takes bf16 rows only", dtype);
  if (!dw) return fail(BMOE_ERR_NULL, "dw is NULL");
  if (rows > 0 && (!dz || !u)) return fail(BMOE_ERR_NULL, "dz / u is NULL");
  const size_t need = sgrad_workspace(d_out, d_in, rows);
  if (need > 0 && !workspace) return fail(BMOE_ERR_NULL, "workspace is NULL");
  if (!aligned(dw, 16)) return fail(BMOE_ERR_ALIGN, "dw must be 16-byte aligned");
  if (rows > 0 && (!aligned(dz, 16) || !aligned(u, 16))) return fail(BMOE_ERR_ALIGN, "dz and u must be 16-byte aligned");
  if (need > 0 && !aligned(workspace, 16)) return fail(BMOE_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(BMOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  const Range rw{dw, size_t(d_out) * d_in * 4}, rz{dz, size_t(rows) * d_out * 2}, ru{u, size_t(rows) * d_in * 2},
      rws{workspace, need};
  if ((rows > 0 && (overlap(rw, rz) || overlap(rw, ru))) || overlap(rw, rws))
    return fail(BMOE_ERR_ALIAS, "dw overlaps an input or the workspace");
  if (need > 0 && rows > 0 && (overlap(rws, rz) || overlap(rws, ru)))
    return fail(BMOE_ERR_ALIAS, "the workspace overlaps an input");
  st = check_device();
  if (st != BMOE_OK) return st;
  BMOE_HIP(launch_sgrad(dz, u, alpha, dw, static_cast<float*>(workspace), rows, d_out, d_in, stream));
  return ok();
}

// ---------------------------------------------------------------- combine backward
bmoe_status bmoe_combine_backward(int32_t T, int32_t top_k, int32_t d, int32_t dtype, const void* dy,
                                  const int32_t* bucket_slots, const float* topk_gate, const void* o,
                                  void* d_rows, float* d_gate, hipStream_t stream) {
  if (T < 0 || top_k < 1 || top_k > 8 || d < 8 || d > 16384 || d % 8 != 0)
    return fail(BMOE_ERR_SHAPE, "T=%d, top_k=%d, d=%d: need T >= 0, top_k in [1, 8], d a multiple of 8 in [8, 16384]",
                T, top_k, d);
  const int64_t R = int64_t(T) * top_k;
  if (R * d > (int64_t(1) << 31) - 1) return fail(BMOE_ERR_SHAPE, "T * top_k * d must be below 2^31");
  if (dtype != BMOE_F32 && dtype != BMOE_BF16) return fail(BMOE_ERR_DTYPE, "dtype=%d is unknown", dtype);
  if ((o == nullptr) != (d_gate == nullptr)) return fail(BMOE_ERR_NULL, "o and d_gate must be given together");
  if (R > 0 && (!dy || !bucket_slots || !topk_gate || !d_rows)) return fail(BMOE_ERR_NULL, "an input or d_rows is NULL");
  if (R > 0 && (!aligned(dy, 16) || !aligned(d_rows, 16) || (o && !aligned(o, 16))))
    return fail(BMOE_ERR_ALIGN, "dy, o and d_rows must be 16-byte aligned");
  if (R > 0 && (!aligned(bucket_slots, 4) || !aligned(topk_gate, 4) || (d_gate && !aligned(d_gate, 4))))
    return fail(BMOE_ERR_ALIGN, "bucket_slots, topk_gate and d_gate must be 4-byte aligned");
  const size_t es = dtype == BMOE_BF16 ? 2 : 4;
  const Range rdy{dy, size_t(T) * d * es}, rsl{bucket_slots, size_t(R) * 4}, rg{topk_gate, size_t(R) * 4},
      ro{o, o ? size_t(R) * d * es : 0}, rr{d_rows, size_t(R) * d * es}, rdg{d_gate, d_gate ? size_t(R) * 4 : 0};
  if (R > 0 && (overlap(rr, rdy) || overlap(rr, rsl) || overlap(rr, rg) || overlap(rr, ro) || overlap(rr, rdg)))
    return fail(BMOE_ERR_ALIAS, "d_rows overlaps an input or d_gate");
  if (R > 0 && d_gate && (overlap(rdg, rdy) || overlap(rdg, rsl) || overlap(rdg, rg) || overlap(rdg, ro)))
    return fail(BMOE_ERR_ALIAS, "d_gate overlaps an input");
  const bmoe_status st = check_device();
  if (st != BMOE_OK) return st;
  BMOE_HIP(launch_combine_bwd(dy, bucket_slots, topk_gate, o, d_rows, d_gate, int(R), top_k, d,
                              dtype == BMOE_BF16 ? ACT_BF16 : ACT_F32, stream));
  return ok();
}

// ---------------------------------------------------------------- router backward
static bmoe_status check_rbwd_shape(int32_t T, int32_t d, int32_t N) {
  if (T < 0 || d < 8 || d > 2048 || d % 8 != 0 || N < 1 || N > 256)
    return fail(BMOE_ERR_SHAPE, "T=%d, d=%d, N=%d: need T >= 0, d a multiple of 8 in [8, 2048], N in [1, 256]", T,
                d, N);
  if (int64_t(T) * (d > N ? d : N) > (int64_t(1) << 31) - 1) return fail(BMOE_ERR_SHAPE, "T * max(d, N) beyond 2^31");
  return BMOE_OK;
}

bmoe_status bmoe_router_backward_workspace(int32_t T, int32_t d, int32_t n_experts, size_t* bytes) {
  if (!bytes) return fail(BMOE_ERR_NULL, "bytes is NULL");
  const bmoe_status st = check_rbwd_shape(T, d, n_experts);
  if (st != BMOE_OK) return st;
  *bytes = router_bwd_workspace(T, d, n_experts);
  return ok();
}

bmoe_status bmoe_router_backward(int32_t T, int32_t d, int32_t n_experts, int32_t top_k, int32_t renorm_gates,
                                 int32_t dtype, const void* x, const void* w_gate, const int32_t* topk_idx,
                                 const float* d_gate, float* dx, float* dw_gate, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  bmoe_status st = check_rbwd_shape(T, d, n_experts);
  if (st != BMOE_OK) return st;
  if (top_k < 1 || top_k > 8 || top_k > n_experts) return fail(BMOE_ERR_SHAPE, "top_k=%d must be in [1, min(8, N)]", top_k);
  if (renorm_gates != 0 && renorm_gates != 1) return fail(BMOE_ERR_SHAPE, "renorm_gates must be 0 or 1");
  if (dtype != BMOE_F32 && dtype != BMOE_BF16) return fail(BMOE_ERR_DTYPE, "dtype=%d is unknown", dtype);
  if (!w_gate || !dw_gate) return fail(BMOE_ERR_NULL, "w_gate / dw_gate is NULL");
  if (T > 0 && (!x || !topk_idx || !d_gate || !dx)) return fail(BMOE_ERR_NULL, "x / topk_idx / d_gate / dx is NULL");
  const size_t need = router_bwd_workspace(T, d, n_experts);
  if (need > 0 && !workspace) return fail(BMOE_ERR_NULL, "workspace is NULL");
  if (!aligned(w_gate, 16) || !aligned(dw_gate, 4) || (T > 0 && (!aligned(x, 16) || !aligned(dx, 4))))
    return fail(BMOE_ERR_ALIGN, "x and w_gate must be 16-byte aligned, dx and dw_gate 4-byte aligned");
  if (T > 0 && (!aligned(topk_idx, 4) || !aligned(d_gate, 4)))
    return fail(BMOE_ERR_ALIGN, "topk_idx and d_gate must be 4-byte aligned");
  if (need > 0 && !aligned(workspace, 16)) return fail(BMOE_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(BMOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  const size_t es = dtype == BMOE_BF16 ? 2 : 4;
  const Range rx{x, size_t(T) * d * es}, rw{w_gate, size_t(n_experts) * d * es}, ri{topk_idx, size_t(T) * top_k * 4},
      rg{d_gate, size_t(T) * top_k * 4}, rdx{dx, size_t(T) * d * 4}, rdw{dw_gate, size_t(n_experts) * d * 4},
      rws{workspace, need};
  if (overlap(rdw, rw) || overlap(rdw, rws) ||
      (T > 0 && (overlap(rdw, rx) || overlap(rdw, ri) || overlap(rdw, rg) || overlap(rdw, rdx))))
    return fail(BMOE_ERR_ALIAS, "dw_gate overlaps an input, dx or the workspace");
  if (T > 0 && (overlap(rdx, rx) || overlap(rdx, rw) || overlap(rdx, ri) || overlap(rdx, rg) || overlap(rdx, rws)))
    return fail(BMOE_ERR_ALIAS, "dx overlaps an input or the workspace");
  if (need > 0 && (overlap(rws, rw) || (T > 0 && (overlap(rws, rx) || overlap(rws, ri) || overlap(rws, rg)))))
    return fail(BMOE_ERR_ALIAS, "the workspace overlaps an input");
  st = check_device();
  if (st != BMOE_OK) return st;
  BMOE_HIP(launch_router_bwd(x, w_gate, topk_idx, d_gate, dx, dw_gate, workspace, T, d, n_experts, top_k,
                             renorm_gates, dtype == BMOE_BF16 ? ACT_BF16 : ACT_F32, stream));
  return ok();
}

// ---------------------------------------------------------------- GELU derivative
bmoe_status bmoe_gelu_backward(int32_t rows, int32_t width, int32_t dtype, const void* h, const void* da, void* dh,
                               hipStream_t stream) {
  if (rows < 0 || width < 8 || width % 8 != 0 || int64_t(rows) * width > (int64_t(1) << 31) - 1)
    return fail(BMOE_ERR_SHAPE, "rows=%d, width=%d: need rows >= 0, width a multiple of 8, rows * width below 2^31",
                rows, width);
  if (dtype != BMOE_F32 && dtype != BMOE_BF16) return fail(BMOE_ERR_DTYPE, "dtype=%d is unknown", dtype);
  if (rows == 0) return ok();
  if (!h || !da || !dh) return fail(BMOE_ERR_NULL, "h / da / dh is NULL");
  if (!aligned(h, 16) || !aligned(da, 16) || !aligned(dh, 16)) return fail(BMOE_ERR_ALIGN, "h, da and dh must be 16-byte aligned");
  const size_t bytes = size_t(rows) * width * (dtype == BMOE_BF16 ? 2 : 4);
  const Range rh{h, bytes}, rd{da, bytes}, ro{dh, bytes};
  if ((dh != h && overlap(ro, rh)) || (dh != da && overlap(ro, rd)))
    return fail(BMOE_ERR_ALIAS, "dh overlaps h or da without being the same buffer");
  const bmoe_status st = check_device();
  if (st != BMOE_OK) return st;
  BMOE_HIP(launch_gelu_bwd(h, da, dh, size_t(rows) * width, dtype == BMOE_BF16 ? ACT_BF16 : ACT_F32, stream));
  return ok();
}

// ---------------------------------------------------------------- substrate input gradient
bmoe_status bmoe_substrate_input_grad(int32_t rows, int32_t d_out, int32_t d_in, int32_t dtype, const void* dz,
                                      const uint32_t* wt_packed, float alpha, void* du, hipStream_t stream) {
  if (dtype != BMOE_F32 && dtype != BMOE_BF16) return fail(BMOE_ERR_DTYPE, "dtype=%d is unknown", dtype);
  const int q = dtype == BMOE_BF16 ? 64 : 16;
  if (rows < 0 || d_out < q || d_in < q || d_out % q || d_in % q)
    return fail(BMOE_ERR_SHAPE, "rows=%d d_out=%d d_in=%d: d_out and d_in must be positive multiples of %d", rows,
                d_out, d_in, q);
  if (int64_t(rows) * (d_out > d_in ? d_out : d_in) > (int64_t(1) << 31) - 1)
    return fail(BMOE_ERR_SHAPE, "rows * max(d_out, d_in) must be below 2^31");
  if (rows == 0) return ok();
  if (!dz || !wt_packed || !du) return fail(BMOE_ERR_NULL, "dz / wt_packed / du is NULL");
  if (!aligned(dz, 16) || !aligned(wt_packed, 16) || !aligned(du, 16))
    return fail(BMOE_ERR_ALIGN, "dz, wt_packed and du must be 16-byte aligned");
  const size_t s = dtype == BMOE_BF16 ? 2 : 4;
  const Range rz{dz, size_t(rows) * d_out * s}, ru{du, size_t(rows) * d_in * s},
      rw{wt_packed, size_t(d_in) * (d_out / 16) * 4};
  if (overlap(ru, rz) || overlap(ru, rw)) return fail(BMOE_ERR_ALIAS, "du overlaps dz or the packed substrate");
  const bmoe_status st = check_device();
  if (st != BMOE_OK) return st;
  GemmArgs g{dz, wt_packed, du, alpha, rows, d_in, d_out};
  BMOE_HIP(launch_gemm(g, dtype == BMOE_BF16 ? ACT_BF16 : ACT_F32, stream));
  return ok();
}

// ---------------------------------------------------------------- training path
namespace {

// State of a training forward (slices 256-byte aligned): routing, then the rows
// the backward reads, in bucket order and the activation dtype.
struct TrainLayout {
  size_t idx, gate, offsets, perm, qpos, U, H1, H, V, Z, O, total;
};

TrainLayout train_layout(const bmoe_layer* L, int32_t T) {
  TrainLayout t{};
  const size_t R = size_t(T) * L->top_k, s = act_size(L->act_dtype);
  const size_t d = size_t(L->d_model), f = size_t(L->d_ff);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  t.idx = take(R * 4);
  t.gate = take(R * 4);
  t.offsets = take(size_t(L->n_experts + 1) * 4);
  t.perm = take(R * 4);
  t.qpos = take(R * 4);
  t.U = take(R * d * s);
  if (f) {
    t.H1 = take(R * f * s);
    t.H = take(R * f * s);
    t.V = take(R * f * s);
  }
  t.Z = take(R * d * s);
  t.O = take(R * d * s);
  t.total = o;
  return t;
}

// Workspace of the training forward: the router's tile lists, and at FFN
// layers the GELU output between the two middle rotations.
struct TrainFwdWs {
  size_t tslots, tgates, tstart, A, total;
  int32_t tiles;
};

TrainFwdWs train_fwd_ws(const bmoe_layer* L, int32_t T) {
  TrainFwdWs w{};
  const size_t R = size_t(T) * L->top_k;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  w.tiles = T > 0 ? int32_t((int64_t(T) + router_tile(T, L) - 1) / router_tile(T, L)) : 0;
  w.tslots = take(R * 4);
  w.tgates = take(R * 4);
  w.tstart = take(size_t(w.tiles) * L->n_experts * 4);
  w.A = take(L->d_ff ? R * size_t(L->d_ff) * act_size(L->act_dtype) : 0);
  w.total = o;
  return w;
}

// Workspace of the layer backward (see bmoe_layer_backward for the data flow).
struct TrainBwdWs {
  size_t G1, G2, A, xb, c1, c2, dgate, dxr, wt0, wt1, bb, sg, rb, total;
};

TrainBwdWs train_bwd_ws(const bmoe_layer* L, int32_t T) {
  TrainBwdWs w{};
  const int32_t R = T * L->top_k;
  const size_t s = act_size(L->act_dtype);
  const size_t d = size_t(L->d_model), f = size_t(L->d_ff), wide = f > d ? f : d;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  w.G1 = take(size_t(R) * wide * s);
  w.G2 = take(size_t(R) * wide * s);
  w.A = take(f ? size_t(R) * f * s : 0);
  w.xb = take(size_t(R) * d * s);
  const bool cast = L->act_dtype != BMOE_BF16;  // the substrate gradient takes bf16 rows
  w.c1 = take(cast ? size_t(R) * wide * 2 : 0);
  w.c2 = take(cast ? size_t(R) * wide * 2 : 0);
  w.dgate = take(size_t(R) * 4);
  w.dxr = take(size_t(T) * d * 4);
  int32_t n0, k0, n1 = 0, k1 = 0;
  sub_shape(L, 0, n0, k0);
  if (f) sub_shape(L, 1, n1, k1);
  w.wt0 = take(size_t(n0) * k0 / 4);
  w.wt1 = take(f ? size_t(n1) * k1 / 4 : 0);
  size_t bb = bfly_bwd_workspace(ilog2(L->d_model), L->n_experts, R);
  if (f) {
    const size_t bf = bfly_bwd_workspace(ilog2(L->d_ff), L->n_experts, R);
    bb = bf > bb ? bf : bb;
  }
  w.bb = take(bb);
  size_t sg = sgrad_workspace(n0, k0, R);
  if (f) {
    const size_t s1 = sgrad_workspace(n1, k1, R);
    sg = s1 > sg ? s1 : sg;
  }
  w.sg = take(sg);
  w.rb = take(router_bwd_workspace(T, L->d_model, L->n_experts));
  w.total = o;
  return w;
}

bmoe_status check_train_layer(const bmoe_layer* L, int32_t T) {
  bmoe_status st = check_layer(L);
  if (st != BMOE_OK) return st;
  if (T < 0 || T > kMaxTokens) return fail(BMOE_ERR_SHAPE, "T=%d must be in [0, %d]", T, kMaxTokens);
  if (L->d_model < 128 || (L->d_ff && L->d_ff < 128))
    return fail(BMOE_ERR_SHAPE, "the training path needs d_model and d_ff of at least 128 (d_model=%d, d_ff=%d)",
                L->d_model, L->d_ff);
  if (L->d_model > 2048) return fail(BMOE_ERR_SHAPE, "the training path's router backward takes d_model <= 2048");
  const int64_t R = int64_t(T) * L->top_k, wide = L->d_ff > L->d_model ? L->d_ff : L->d_model;
  if (R * wide > (int64_t(1) << 31) - 1) return fail(BMOE_ERR_SHAPE, "T * top_k * max(d_model, d_ff) beyond 2^31");
  return BMOE_OK;
}

}  // namespace

extern "C" {

bmoe_status bmoe_train_state_size(const bmoe_layer* layer, int32_t T, size_t* bytes) {
  if (!bytes) return fail(BMOE_ERR_NULL, "bytes is NULL");
  const bmoe_status st = check_train_layer(layer, T);
  if (st != BMOE_OK) return st;
  *bytes = train_layout(layer, T).total;
  return ok();
}

bmoe_status bmoe_forward_train_workspace(const bmoe_layer* layer, int32_t T, size_t* bytes) {
  if (!bytes) return fail(BMOE_ERR_NULL, "bytes is NULL");
  const bmoe_status st = check_train_layer(layer, T);
  if (st != BMOE_OK) return st;
  *bytes = train_fwd_ws(layer, T).total;
  return ok();
}

bmoe_status bmoe_layer_backward_workspace(const bmoe_layer* layer, int32_t T, size_t* bytes) {
  if (!bytes) return fail(BMOE_ERR_NULL, "bytes is NULL");
  const bmoe_status st = check_train_layer(layer, T);
  if (st != BMOE_OK) return st;
  *bytes = train_bwd_ws(layer, T).total;
  return ok();
}

// Training forward: route and bucket as bmoe_forward; then, per routed row in
// bucket order, U = B(theta_0)^T x_t (gathered), square: Z = alpha U W^T;
// FFN: H1 = alpha U W_up^T, H = B(phi_up) H1, A = act(H) (workspace),
// V = B(theta_dn)^T A, Z = alpha V W_dn^T; O = B(phi_last) Z; y_t = sum_j of
// the gated rows in slot order.
bmoe_status bmoe_forward_train(const bmoe_layer* layer, const void* x, int32_t T, void* y, void* state,
                               size_t state_bytes, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  bmoe_status st = check_train_layer(layer, T);
  if (st != BMOE_OK) return st;
  const TrainLayout tl = train_layout(layer, T);
  const TrainFwdWs fw = train_fwd_ws(layer, T);
  if (T == 0) return ok();
  if (!x || !y || !state || !workspace) return fail(BMOE_ERR_NULL, "x / y / state / workspace is NULL");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(state, 256) || !aligned(workspace, 256))
    return fail(BMOE_ERR_ALIGN, "x and y must be 16-byte aligned, state and workspace 256-byte aligned");
  if (state_bytes < tl.total) return fail(BMOE_ERR_WORKSPACE, "state has %zu bytes, %zu needed", state_bytes, tl.total);
  if (workspace_bytes < fw.total)
    return fail(BMOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, fw.total);
  const size_t s = act_size(layer->act_dtype);
  const Range rx{x, size_t(T) * layer->d_model * s}, ry{y, size_t(T) * layer->d_model * s},
      rs{state, tl.total}, rw{workspace, fw.total};
  if (overlap(ry, rx) || overlap(ry, rs) || overlap(ry, rw)) return fail(BMOE_ERR_ALIAS, "y overlaps x, the state or the workspace");
  if (overlap(rs, rx) || overlap(rs, rw) || overlap(rw, rx))
    return fail(BMOE_ERR_ALIAS, "the state, the workspace and x must not overlap");
  st = check_device();
  if (st != BMOE_OK) return st;

  const int act = layer->act_dtype == BMOE_BF16 ? ACT_BF16 : ACT_F32;
  const int32_t N = layer->n_experts, k = layer->top_k, d = layer->d_model, f = layer->d_ff;
  const int32_t R = T * k;
  int32_t* idx = at<int32_t>(state, tl.idx);
  float* gate = at<float>(state, tl.gate);
  int32_t* offsets = at<int32_t>(state, tl.offsets);
  int32_t* perm = at<int32_t>(state, tl.perm);
  int32_t* qpos = at<int32_t>(state, tl.qpos);
  void* U = at<char>(state, tl.U);
  void* Z = at<char>(state, tl.Z);
  void* O = at<char>(state, tl.O);
  RouteArgs ra{x, layer->w_gate, idx, gate, T, d, N, k, layer->renorm_gates,
               at<int32_t>(workspace, fw.tslots), at<float>(workspace, fw.tgates), at<int32_t>(workspace, fw.tstart)};
  BMOE_HIP(launch_route(ra, act, stream));
  BucketArgs ba{ra.tile_slots, ra.tile_gates, ra.tile_start, offsets, perm, nullptr, R, N,
                router_tile(T, layer) * k, fw.tiles, 0, 0};
  BMOE_HIP(launch_bucket(ba, stream));
  BMOE_HIP(launch_invert_perm(perm, qpos, R, stream));
  BflyArgs bi{x, U, layer->theta[0], nullptr, offsets, perm, nullptr, R, N, k, 0, 0};
  BMOE_HIP(launch_butterfly(bi, BFLY_IN, act, ilog2(d), stream));
  const void* zin = U;
  if (f) {
    void* H1 = at<char>(state, tl.H1);
    void* H = at<char>(state, tl.H);
    void* V = at<char>(state, tl.V);
    void* A = at<char>(workspace, fw.A);
    BMOE_HIP(launch_gemm(GemmArgs{U, layer->w_base[0], H1, layer->w_scale[0], R, f, d}, act, stream));
    BflyArgs bu{H1, H, layer->phi[0], nullptr, offsets, perm, nullptr, R, N, k, 0, 0};
    BMOE_HIP(launch_bfly_rot(bu, act, ilog2(f), false, stream));
    const void* a_in = H;  // no activation: the rotation reads H itself
    if (layer->ffn_act == BMOE_ACT_GELU_ERF) {
      BMOE_HIP(launch_gelu_fwd(H, A, size_t(R) * f, act, stream));
      a_in = A;
    }
    BflyArgs bd{a_in, V, layer->theta[1], nullptr, offsets, perm, nullptr, R, N, k, 1, 0};
    BMOE_HIP(launch_bfly_rot(bd, act, ilog2(f), true, stream));
    zin = V;
  }
  const int m = f ? 1 : 0;
  int32_t n_out, k_in;
  sub_shape(layer, m, n_out, k_in);
  BMOE_HIP(launch_gemm(GemmArgs{zin, layer->w_base[m], Z, layer->w_scale[m], R, n_out, k_in}, act, stream));
  BflyArgs bo{Z, O, layer->phi[m], nullptr, offsets, perm, nullptr, R, N, k, 0, 0};
  BMOE_HIP(launch_bfly_rot(bo, act, ilog2(d), false, stream));
  BMOE_HIP(launch_token_sum(O, qpos, gate, nullptr, y, false, T, d, k, act, stream));
  return ok();
}

// Layer backward.  Rows in bucket order; G1 / G2 are row-gradient buffers of
// the activation dtype.  With l the last substrate (0 square, 1 FFN):
//   G1 = gate * dy_t (combine backward, with dgate = dy_t . O)
//   G1 = dZ, dphi_l           (output rotation backward, in place)
//   square: G2 = dU = alpha dZ W;  dW_0 = alpha sum dZ^T U
//   FFN:    G2 = dV = alpha dZ W_dn;  dW_1 = alpha sum dZ^T V;  A = act(H)
//           G2 = dA, dtheta_dn (rotation backward, in place);  G2 = dH = act'(H) dA
//           G2 = dH1, dphi_up (in place);  G1 = dU = alpha dH1 W_up;  dW_0 = alpha sum dH1^T U
//   xb = x_t gathered;  dU's buffer = dxb, dtheta_0 (in place)
//   dx_r, dW_g = router backward (x, W_g, idx, dgate);  dx_t = dx_r + sum_j dxb (slot order)
bmoe_status bmoe_layer_backward(const bmoe_layer* layer, const void* x, int32_t T, const void* dy,
                                const void* state, size_t state_bytes, const bmoe_layer_grads* g, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  bmoe_status st = check_train_layer(layer, T);
  if (st != BMOE_OK) return st;
  if (!g) return fail(BMOE_ERR_NULL, "grads is NULL");
  const bool ffn = layer->d_ff != 0;
  const int nm = ffn ? 2 : 1;
  if (!g->d_w_gate) return fail(BMOE_ERR_NULL, "grads->d_w_gate is NULL");
  for (int m = 0; m < nm; ++m)
    if (!g->d_theta[m] || !g->d_phi[m] || !g->d_w_base[m])
      return fail(BMOE_ERR_NULL, "grads->d_theta / d_phi / d_w_base [%d] is NULL", m);
  const TrainLayout tl = train_layout(layer, T);
  const TrainBwdWs bw = train_bwd_ws(layer, T);
  const int32_t N = layer->n_experts, k = layer->top_k, d = layer->d_model, f = layer->d_ff;
  const size_t s = act_size(layer->act_dtype);
  // outputs: ranges, alignment, no overlap with each other or the inputs
  std::vector<Range> outs;
  outs.push_back(Range{g->d_w_gate, size_t(N) * d * 4});
  for (int m = 0; m < nm; ++m) {
    int32_t n_out, k_in;
    sub_shape(layer, m, n_out, k_in);
    outs.push_back(Range{g->d_theta[m], size_t(N) * ilog2(k_in) * (k_in / 2) * 4});
    outs.push_back(Range{g->d_phi[m], size_t(N) * ilog2(n_out) * (n_out / 2) * 4});
    outs.push_back(Range{g->d_w_base[m], size_t(n_out) * k_in * 4});
  }
  if (T > 0) outs.push_back(Range{g->dx, size_t(T) * d * 4});
  for (const Range& r : outs)
    if (!aligned(r.p, 16)) return fail(BMOE_ERR_ALIGN, "gradient outputs must be 16-byte aligned");
  if (T > 0) {
    if (!x || !dy || !state || !workspace || !g->dx) return fail(BMOE_ERR_NULL, "x / dy / state / workspace / dx is NULL");
    if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(state, 256) || !aligned(workspace, 256))
      return fail(BMOE_ERR_ALIGN, "x and dy must be 16-byte aligned, state and workspace 256-byte aligned");
    if (state_bytes < tl.total) return fail(BMOE_ERR_WORKSPACE, "state has %zu bytes, %zu needed", state_bytes, tl.total);
    if (workspace_bytes < bw.total)
      return fail(BMOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, bw.total);
    const Range ins[] = {Range{x, size_t(T) * d * s}, Range{dy, size_t(T) * d * s}, Range{state, tl.total},
                         Range{workspace, bw.total}};
    for (const Range& a : ins)
      for (const Range& b : outs)
        if (overlap(a, b)) return fail(BMOE_ERR_ALIAS, "a gradient output overlaps an input, the state or the workspace");
    if (overlap(ins[3], ins[0]) || overlap(ins[3], ins[1]) || overlap(ins[3], ins[2]))
      return fail(BMOE_ERR_ALIAS, "the workspace overlaps x, dy or the state");
  }
  for (size_t i = 0; i < outs.size(); ++i)
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlap(outs[i], outs[j])) return fail(BMOE_ERR_ALIAS, "two gradient outputs overlap");
  st = check_device();
  if (st != BMOE_OK) return st;
  const int act = layer->act_dtype == BMOE_BF16 ? ACT_BF16 : ACT_F32;
  const int32_t R = T * k;
  if (T == 0) {
    // no rows: every parameter gradient is zero
    for (const Range& r : outs) BMOE_HIP(launch_zero(const_cast<void*>(r.p), r.bytes, stream));
    return ok();
  }
  const int32_t* idx = at<const int32_t>(const_cast<void*>(state), tl.idx);
  const float* gate = at<const float>(const_cast<void*>(state), tl.gate);
  const int32_t* offsets = at<const int32_t>(const_cast<void*>(state), tl.offsets);
  const int32_t* perm = at<const int32_t>(const_cast<void*>(state), tl.perm);
  const int32_t* qpos = at<const int32_t>(const_cast<void*>(state), tl.qpos);
  auto srow = [&](size_t off) { return at<char>(const_cast<void*>(state), off); };
  void* G1 = at<char>(workspace, bw.G1);
  void* G2 = at<char>(workspace, bw.G2);
  float* dgate = at<float>(workspace, bw.dgate);
  float* bbws = at<float>(workspace, bw.bb);
  float* sgws = at<float>(workspace, bw.sg);
  // the substrate gradient takes bf16 rows: fp32 layers cast both operands first
  auto substrate_grad = [&](const void* dz, const void* u, int32_t d_out, int32_t d_in, float alpha,
                            float* out) -> hipError_t {
    const void *a = dz, *b = u;
    if (act != ACT_BF16) {
      uint16_t* c1 = at<uint16_t>(workspace, bw.c1);
      uint16_t* c2 = at<uint16_t>(workspace, bw.c2);
      hipError_t e = launch_cast_bf16(static_cast<const float*>(dz), c1, size_t(R) * d_out, stream);
      if (e != hipSuccess) return e;
      e = launch_cast_bf16(static_cast<const float*>(u), c2, size_t(R) * d_in, stream);
      if (e != hipSuccess) return e;
      a = c1;
      b = c2;
    }
    return launch_sgrad(a, b, alpha, out, sgws, R, d_out, d_in, stream);
  };
  const int m = ffn ? 1 : 0;
  BMOE_HIP(launch_combine_bwd(dy, perm, gate, srow(tl.O), G1, dgate, R, k, d, act, stream));
  BMOE_HIP(launch_bfly_bwd(srow(tl.Z), G1, G1, layer->phi[m], offsets, bbws, g->d_phi[m], R, N, ilog2(d), 0, act,
                           stream));
  void* dU;
  if (!ffn) {
    uint32_t* wt = at<uint32_t>(workspace, bw.wt0);
    BMOE_HIP(launch_transpose_packed(layer->w_base[0], wt, d, d, stream));
    BMOE_HIP(launch_gemm(GemmArgs{G1, wt, G2, layer->w_scale[0], R, d, d}, act, stream));
    BMOE_HIP(substrate_grad(G1, srow(tl.U), d, d, layer->w_scale[0], g->d_w_base[0]));
    dU = G2;
  } else {
    uint32_t* wt1 = at<uint32_t>(workspace, bw.wt1);
    uint32_t* wt0 = at<uint32_t>(workspace, bw.wt0);
    void* A = at<char>(workspace, bw.A);
    BMOE_HIP(launch_transpose_packed(layer->w_base[1], wt1, d, f, stream));    // W_dn [d][f] -> [f][d]
    BMOE_HIP(launch_gemm(GemmArgs{G1, wt1, G2, layer->w_scale[1], R, f, d}, act, stream));  // dV [R][f]
    BMOE_HIP(substrate_grad(G1, srow(tl.V), d, f, layer->w_scale[1], g->d_w_base[1]));
    const bool gelu = layer->ffn_act == BMOE_ACT_GELU_ERF;
    const void* a_in = srow(tl.H);  // no activation: the rotation's input is H itself
    if (gelu) {
      BMOE_HIP(launch_gelu_fwd(srow(tl.H), A, size_t(R) * f, act, stream));
      a_in = A;
    }
    BMOE_HIP(launch_bfly_bwd(a_in, G2, G2, layer->theta[1], offsets, bbws, g->d_theta[1], R, N, ilog2(f), 1, act,
                             stream));
    if (gelu) BMOE_HIP(launch_gelu_bwd(srow(tl.H), G2, G2, size_t(R) * f, act, stream));
    BMOE_HIP(launch_bfly_bwd(srow(tl.H1), G2, G2, layer->phi[0], offsets, bbws, g->d_phi[0], R, N, ilog2(f), 0,
                             act, stream));
    BMOE_HIP(launch_transpose_packed(layer->w_base[0], wt0, f, d, stream));    // W_up [f][d] -> [d][f]
    BMOE_HIP(launch_gemm(GemmArgs{G2, wt0, G1, layer->w_scale[0], R, d, f}, act, stream));  // dU [R][d]
    BMOE_HIP(substrate_grad(G2, srow(tl.U), f, d, layer->w_scale[0], g->d_w_base[0]));
    dU = G1;
  }
  void* xb = at<char>(workspace, bw.xb);
  BMOE_HIP(launch_gather_rows(x, perm, xb, R, d, k, act, stream));
  BMOE_HIP(launch_bfly_bwd(xb, dU, dU, layer->theta[0], offsets, bbws, g->d_theta[0], R, N, ilog2(d), 1, act,
                           stream));
  float* dxr = at<float>(workspace, bw.dxr);
  BMOE_HIP(launch_router_bwd(x, layer->w_gate, idx, dgate, dxr, g->d_w_gate, at<char>(workspace, bw.rb), T, d, N, k,
                             layer->renorm_gates, act, stream));
  BMOE_HIP(launch_token_sum(dU, qpos, nullptr, dxr, g->dx, true, T, d, k, act, stream));
  return ok();
}

}  // extern "C"
