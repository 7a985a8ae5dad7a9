// C ABI of libmoe: host-side validation, block-size choice, workspace layout and the
// launch sequence.  Every check runs before the first HIP call of an entry point, so
// a rejected call enqueues nothing.
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "moe_internal.h"
#include "moe_route.h"

using namespace moe;

namespace {

constexpr int64_t kI32Max = 2147483647LL;

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

int elt_bytes(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1; }

bool is_mx(const moe_problem* p) { return p->dtype == MOE_E4M3 && p->w_dtype == MOE_MXFP4; }

// Rows per m-block for m expected slots per expert.  Few slots per expert: the m-block should
// hold a whole expert so each weight tile is streamed from HBM once; many slots: large
// m-blocks keep the MFMA tiles large (fewer bytes per flop through LDS; the padding of an
// expert's last block grows with the block).  The bf16 thresholds are where the measured
// best block size changes in a batch sweep with uniform routing over 16 experts of
// H = I = 2880 (16 up to 10 slots, 32 up to 28, 64 up to 64, 128 up to 128, then 256).
int32_t block_m_for(double m, int dtype, int w_dtype) {
  // MXFP4 x e4m3: the 64-row kernel (three workgroups per CU) is within 4% of the smaller
  // blocks at every measured size; past 128 slots per expert the 128-row one is as fast or
  // faster (batch sweeps of one GPT-OSS-shaped shard keyed on its own counts, uniform and
  // production-like routing: 64-row blocks win up to 3584 tokens on the latter)
  if (w_dtype == MOE_MXFP4) return m <= 128 ? 64 : 128;
  if (dtype == MOE_BF16 && w_dtype == MOE_BF16) {
    if (m <= 10) return 16;
    if (m <= 28) return 32;
    if (m <= 64) return 64;
    if (m <= 128) return 128;
    return 256;
  }
  if (m <= 8) return 16;
  if (m <= 20) return 32;
  if (m <= 40) return 64;
  return 128;
}

int32_t choose_block_m(const moe_problem* p) {
  if (p->block_m) return p->block_m;
  return block_m_for((double)p->T * p->top_k / p->E, p->dtype, p->w_dtype);
}

int validate(const moe_problem* p) {
  if (!p) return MOE_ERR_NULL;
  if (p->T < 1 || p->E < 1 || p->E > 1024 || p->top_k < 1 || p->top_k > p->E) return MOE_ERR_SHAPE;
  // H and I: multiples of 64 (whole 64-wide k-slices and n-blocks); e4m3 needs 128 (one
  // scale block per 128 values)
  if (p->H < 64 || p->I < 64 || p->H % 64 || p->I % 64) return MOE_ERR_SHAPE;
  if (p->w_dtype == MOE_E4M3 && (p->H % 128 || p->I % 128)) return MOE_ERR_SHAPE;
  if (p->H > kMaxDim || p->I > kMaxDim) return MOE_ERR_SHAPE;
  if (p->block_m != 0 && p->block_m != 16 && p->block_m != 32 && p->block_m != 64 &&
      p->block_m != 128 && p->block_m != 256)
    return MOE_ERR_SHAPE;
  const bool f32 = p->dtype == MOE_F32 && p->w_dtype == MOE_F32;
  const bool bf16 = p->dtype == MOE_BF16 && p->w_dtype == MOE_BF16;
  const bool fp8 = p->dtype == MOE_BF16 && p->w_dtype == MOE_E4M3;
  if (!(f32 || bf16 || fp8 || is_mx(p))) return MOE_ERR_DTYPE;
  if (p->block_m == 256 && !bf16) return MOE_ERR_SHAPE;     // 256-row blocks: bf16 only
  const int64_t N = (int64_t)p->T * p->top_k;
  const int64_t BM = choose_block_m(p);
  const int64_t rows = N + (int64_t)(p->E < N ? p->E : N) * (BM - 1);
  const int64_t slab = is_mx(p) ? (int64_t)p->I * p->H : (int64_t)2 * p->I * p->H * elt_bytes(p->w_dtype);
  if (N > kI32Max || rows > kI32Max) return MOE_ERR_SHAPE;
  if (slab > kI32Max) return MOE_ERR_SHAPE;                                   // one expert slab
  if ((int64_t)p->T * p->H > kI32Max || rows * p->I > kI32Max * 4 || N * p->H > kI32Max * 4)
    return MOE_ERR_SHAPE;
  // grid bound of the GEMM launches
  const int64_t tiles = rows / BM;
  const int64_t nb = (p->I > p->H ? p->I : p->H) / 64;
  if (tiles * nb > kI32Max) return MOE_ERR_SHAPE;
  return MOE_OK;
}

Resolved resolve(const moe_problem* p) {
  Resolved r;
  r.T = p->T; r.H = p->H; r.I = p->I; r.E = p->E; r.K = p->top_k;
  r.BM = choose_block_m(p);
  r.dtype = p->dtype; r.w_dtype = p->w_dtype;
  r.N = (int64_t)p->T * p->top_k;
  r.rows_max = r.N + (int64_t)(p->E < r.N ? p->E : r.N) * (r.BM - 1);
  r.tiles_max = r.rows_max / r.BM;
  return r;
}

// Workspace pieces of moe_forward, in order, each 256-byte aligned.
struct Layout {
  int64_t status, counts, offsets, sorted_slots, slot_row, tiles, num_tiles;
  int64_t xq, x_scales, act, act_scales, slot_out, split, total;
};

Layout layout(const Resolved& r) {
  Layout L;
  int64_t o = 0;
  auto take = [&](int64_t bytes) { int64_t at = o; o = align_up(o + bytes, 256); return at; };
  const bool fp8 = r.w_dtype == MOE_E4M3;
  L.status = take(256);
  L.counts = take(4LL * r.E);
  L.offsets = take(4LL * (r.E + 1));
  L.sorted_slots = take(4LL * r.rows_max);
  L.slot_row = take(4LL * r.N);
  L.tiles = take(8LL * r.tiles_max);
  L.num_tiles = take(4);
  L.xq = fp8 ? take((int64_t)r.T * r.H) : -1;
  L.x_scales = fp8 ? take(4LL * r.T * (r.H / kGroup)) : -1;
  L.act = take(r.rows_max * r.I * (fp8 ? 1 : elt_bytes(r.dtype)));
  L.act_scales = fp8 ? take(4LL * r.rows_max * (r.I / kGroup)) : -1;
  L.slot_out = take(r.N * r.H * elt_bytes(r.dtype));
  const int64_t split = gemm_split_bytes(r);
  L.split = split > 0 ? take(split) : -1;
  L.total = o;
  return L;
}

std::mutex g_dev_mu;
int8_t g_dev_ok[64];      // 0 unknown, 1 ok, -1 not gfx950
int g_dev_cus[64];        // compute units, 0 until known

// Library-owned intermediates of moe_forward_scratch: one copy per device, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not the device array, so
// host code never passes it to a kernel or a copy; it uses the device address that
// hipGetSymbolAddress returns for the current device (g_scratch_ptr).
static __device__ __align__(256) char scratch[MOE_SCRATCH_MAX_BYTES];
char* g_scratch_ptr[64];  // device address of `scratch` per device ordinal, null until known

// gfx950 check, cached per device ordinal (with the device's compute-unit count).
int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> g(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_DEVICE;
    g_dev_ok[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_dev_cus[dev] = prop.multiProcessorCount;
  }
  return g_dev_ok[dev] == 1 ? MOE_OK : MOE_ERR_DEVICE;
}

int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

// Device address of this device's `scratch`, looked up once per device with that device
// current (each device holds its own copy at its own address).  Null on failure.
char* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> g(g_dev_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = (char*)p;
  }
  return g_scratch_ptr[dev];
}

// MOE_ERR_ALIGN unless every non-null pointer is aligned to its byte count.
struct Al {
  const void* p;
  int a;
};
int check_align(std::initializer_list<Al> ptrs) {
  for (const Al& x : ptrs)
    if (x.p && ((uintptr_t)x.p & (uintptr_t)(x.a - 1))) return MOE_ERR_ALIGN;
  return MOE_OK;
}

// The launch sequence of moe_forward in the workspace `ws` (device memory of at least
// L.total bytes, 256-byte aligned); n_invalid: where the excluded-slot count goes (null: the
// workspace's first int32).  No piece of the workspace needs to start zeroed: every one is
// written before it is read in the same call.
int forward_in(const Resolved& r, const Layout& L, char* ws, int32_t* n_invalid, const void* x,
               const int32_t* topk_ids, const float* topk_weights, const void* w13,
               const float* w13_scales, const void* w2, const float* w2_scales, void* out,
               hipStream_t s) {
  const bool fp8 = r.w_dtype == MOE_E4M3;
  auto at = [&](int64_t off) { return off < 0 ? nullptr : (void*)(ws + off); };
  if (!n_invalid) n_invalid = (int32_t*)at(L.status);
  int32_t* counts = (int32_t*)at(L.counts);
  int32_t* offsets = (int32_t*)at(L.offsets);
  int32_t* sorted_slots = (int32_t*)at(L.sorted_slots);
  int32_t* slot_row = (int32_t*)at(L.slot_row);
  int32_t* tiles = (int32_t*)at(L.tiles);
  int32_t* num_tiles = (int32_t*)at(L.num_tiles);

  hipError_t e = launch_align(r, topk_ids, counts, offsets, sorted_slots, slot_row, tiles,
                              num_tiles, n_invalid, s);
  if (e != hipSuccess) return MOE_ERR_LAUNCH;
  const void* x_in = x;
  const float* x_scales = nullptr;
  if (fp8) {
    e = launch_quant_rows(r, x, (uint8_t*)at(L.xq), (float*)at(L.x_scales), s);
    if (e != hipSuccess) return MOE_ERR_LAUNCH;
    x_in = at(L.xq);
    x_scales = (const float*)at(L.x_scales);
  }
  e = launch_up(r, x_in, x_scales, w13, w13_scales, sorted_slots, offsets, tiles, num_tiles,
                at(L.act), (float*)at(L.act_scales), at(L.split), s);
  if (e != hipSuccess) return MOE_ERR_LAUNCH;
  e = launch_down(r, at(L.act), (const float*)at(L.act_scales), w2, w2_scales, topk_weights,
                  sorted_slots, offsets, tiles, num_tiles, at(L.slot_out), at(L.split), s);
  if (e != hipSuccess) return MOE_ERR_LAUNCH;
  e = launch_combine(r, at(L.slot_out), slot_row, out, s);
  return status_of(e);
}

}  // namespace

// Every entry point runs check_device() before it launches, so the count is known here;
// 0 (unknown) turns the GEMMs' K-split tail off.
int moe::device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> g(g_dev_mu);
  return g_dev_cus[dev];
}

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: dimension out of range or not a supported multiple";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE: unsupported dtype combination";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH: kernel launch failed";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE: no gfx950 device current";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a device pointer is not aligned as required";
    default: return "unknown moe_status";
  }
}

int moe_validate(const moe_problem* p) { return validate(p); }

int32_t moe_pick_block_m(const moe_problem* p) {
  const int v = validate(p);
  return v != MOE_OK ? v : choose_block_m(p);
}

int32_t moe_block_m_for(double slots_per_expert, int32_t dtype, int32_t w_dtype) {
  const bool ok = (dtype == MOE_F32 && w_dtype == MOE_F32) ||
                  (dtype == MOE_BF16 && (w_dtype == MOE_BF16 || w_dtype == MOE_E4M3)) ||
                  (dtype == MOE_E4M3 && w_dtype == MOE_MXFP4);
  if (!ok) return MOE_ERR_DTYPE;
  if (!(slots_per_expert >= 0.0)) return MOE_ERR_SHAPE;      // negative or NaN
  return block_m_for(slots_per_expert, dtype, w_dtype);
}

int64_t moe_max_padded_slots(const moe_problem* p) {
  const int v = validate(p);
  return v != MOE_OK ? v : resolve(p).rows_max;
}

int64_t moe_max_tiles(const moe_problem* p) {
  const int v = validate(p);
  return v != MOE_OK ? v : resolve(p).tiles_max;
}

int64_t moe_gemm_workspace_bytes(const moe_problem* p) {
  const int v = validate(p);
  if (v != MOE_OK) return v;
  if (is_mx(p)) return MOE_ERR_DTYPE;
  return gemm_split_bytes(resolve(p));
}

int64_t moe_workspace_bytes(const moe_problem* p) {
  const int v = validate(p);
  if (v != MOE_OK) return v;
  if (is_mx(p)) return MOE_ERR_DTYPE;                       // no moe_forward for MXFP4
  return layout(resolve(p)).total;
}

int moe_route(const moe_problem* p, const float* logits, int renormalize, int32_t* topk_ids,
              float* topk_weights, void* stream) {
  int v = validate(p);
  if (v) return v;
  if (p->top_k > kRouteMaxK) return MOE_ERR_SHAPE;
  if (!logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
  if ((v = check_align({{logits, 4}, {topk_ids, 4}, {topk_weights, 4}}))) return v;
  if ((v = check_device())) return v;
  const Resolved r = resolve(p);
  return status_of(launch_route(r, logits, renormalize, topk_ids, topk_weights, (hipStream_t)stream));
}

int moe_route_align(const moe_problem* p, const float* logits, int renormalize, int32_t* topk_ids,
                    float* topk_weights, int32_t* counts, int32_t* offsets, int32_t* sorted_slots,
                    int32_t* slot_row, int32_t* tiles, int32_t* num_tiles, int32_t* n_invalid,
                    void* stream) {
  int v = validate(p);
  if (v) return v;
  if (p->top_k > kRouteMaxK) return MOE_ERR_SHAPE;
  if (!logits || !topk_ids || !topk_weights || !counts || !offsets || !sorted_slots ||
      !slot_row || !tiles || !num_tiles || !n_invalid)
    return MOE_ERR_NULL;
  if ((v = check_align({{logits, 4}, {topk_ids, 4}, {topk_weights, 4}, {counts, 4}, {offsets, 4},
                        {sorted_slots, 4}, {slot_row, 4}, {tiles, 4}, {num_tiles, 4},
                        {n_invalid, 4}})))
    return v;
  if ((v = check_device())) return v;
  const Resolved r = resolve(p);
  return status_of(launch_route_align(r, logits, renormalize, topk_ids, topk_weights, counts,
                                      offsets, sorted_slots, slot_row, tiles, num_tiles,
                                      n_invalid, (hipStream_t)stream));
}

int moe_align(const moe_problem* p, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
              int32_t* sorted_slots, int32_t* slot_row, int32_t* tiles, int32_t* num_tiles,
              int32_t* n_invalid, void* stream) {
  int v = validate(p);
  if (v) return v;
  if (!topk_ids || !counts || !offsets || !sorted_slots || !slot_row || !tiles || !num_tiles ||
      !n_invalid)
    return MOE_ERR_NULL;
  if ((v = check_align({{topk_ids, 4}, {counts, 4}, {offsets, 4}, {sorted_slots, 4},
                        {slot_row, 4}, {tiles, 4}, {num_tiles, 4}, {n_invalid, 4}})))
    return v;
  if ((v = check_device())) return v;
  const Resolved r = resolve(p);
  return status_of(launch_align(r, topk_ids, counts, offsets, sorted_slots, slot_row, tiles,
                                num_tiles, n_invalid, (hipStream_t)stream));
}

int moe_quantize_rows_e4m3(const moe_problem* p, const void* x, uint8_t* xq, float* scales,
                           void* stream) {
  int v = validate(p);
  if (v) return v;
  if (p->w_dtype != MOE_E4M3 || p->dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (!x || !xq || !scales) return MOE_ERR_NULL;
  if ((v = check_align({{x, 16}, {xq, 16}, {scales, 4}}))) return v;
  if ((v = check_device())) return v;
  return status_of(launch_quant_rows(resolve(p), x, xq, scales, (hipStream_t)stream));
}

int moe_grouped_gemm_up(const moe_problem* p, const void* x, const float* x_scales,
                        const void* w13, const float* w13_scales, const int32_t* sorted_slots,
                        const int32_t* offsets, const int32_t* tiles, const int32_t* num_tiles,
                        void* act, float* act_scales, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int v = validate(p);
  if (v) return v;
  if (is_mx(p)) return MOE_ERR_DTYPE;
  if (!x || !w13 || !sorted_slots || !offsets || !tiles || !num_tiles || !act) return MOE_ERR_NULL;
  if (p->w_dtype == MOE_E4M3 && (!x_scales || !w13_scales || !act_scales)) return MOE_ERR_NULL;
  const Resolved r = resolve(p);
  const int64_t split = gemm_split_bytes(r);
  if (workspace && (int64_t)workspace_bytes < split) return MOE_ERR_WORKSPACE;
  if ((v = check_align({{x, 16}, {x_scales, 4}, {w13, 16}, {w13_scales, 4}, {sorted_slots, 4},
                        {offsets, 4}, {tiles, 4}, {num_tiles, 4}, {act, 16}, {act_scales, 4},
                        {workspace, 256}})))
    return v;
  if ((v = check_device())) return v;
  return status_of(launch_up(r, x, x_scales, w13, w13_scales, sorted_slots, offsets, tiles,
                             num_tiles, act, act_scales, split > 0 ? workspace : nullptr,
                             (hipStream_t)stream));
}

int moe_grouped_gemm_up_mxfp4(const moe_problem* p, const uint8_t* x, const float* x_scale,
                              const uint8_t* w13, const uint8_t* w13_scales, const float* bias,
                              float alpha, float limit, const float* out_scale,
                              const int32_t* sorted_slots, const int32_t* offsets,
                              const int32_t* tiles, const int32_t* num_tiles, uint8_t* act,
                              void* stream) {
  int v = validate(p);
  if (v) return v;
  if (!is_mx(p)) return MOE_ERR_DTYPE;
  if (!x || !x_scale || !w13 || !w13_scales || !bias || !out_scale || !sorted_slots ||
      !offsets || !tiles || !num_tiles || !act)
    return MOE_ERR_NULL;
  if ((v = check_align({{x, 16}, {x_scale, 4}, {w13, 16}, {w13_scales, 4}, {bias, 16},
                        {out_scale, 4}, {sorted_slots, 4}, {offsets, 4}, {tiles, 4},
                        {num_tiles, 4}, {act, 16}})))
    return v;
  if ((v = check_device())) return v;
  return status_of(launch_up_mxfp4(resolve(p), x, x_scale, w13, w13_scales, bias, alpha, limit,
                                   out_scale, sorted_slots, offsets, tiles, num_tiles, act,
                                   (hipStream_t)stream));
}

int moe_grouped_gemm_down(const moe_problem* p, const void* act, const float* act_scales,
                          const void* w2, const float* w2_scales, const float* topk_weights,
                          const int32_t* sorted_slots, const int32_t* offsets,
                          const int32_t* tiles, const int32_t* num_tiles, void* slot_out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  int v = validate(p);
  if (v) return v;
  if (is_mx(p)) return MOE_ERR_DTYPE;
  if (!act || !w2 || !topk_weights || !sorted_slots || !offsets || !tiles || !num_tiles ||
      !slot_out)
    return MOE_ERR_NULL;
  if (p->w_dtype == MOE_E4M3 && (!act_scales || !w2_scales)) return MOE_ERR_NULL;
  const Resolved r = resolve(p);
  const int64_t split = gemm_split_bytes(r);
  if (workspace && (int64_t)workspace_bytes < split) return MOE_ERR_WORKSPACE;
  if ((v = check_align({{act, 16}, {act_scales, 4}, {w2, 16}, {w2_scales, 4}, {topk_weights, 4},
                        {sorted_slots, 4}, {offsets, 4}, {tiles, 4}, {num_tiles, 4},
                        {slot_out, 16}, {workspace, 256}})))
    return v;
  if ((v = check_device())) return v;
  return status_of(launch_down(r, act, act_scales, w2, w2_scales, topk_weights, sorted_slots,
                               offsets, tiles, num_tiles, slot_out,
                               split > 0 ? workspace : nullptr, (hipStream_t)stream));
}

int moe_combine(const moe_problem* p, const void* slot_out, const int32_t* slot_row, void* out,
                void* stream) {
  int v = validate(p);
  if (v) return v;
  if (is_mx(p)) return MOE_ERR_DTYPE;
  if (!slot_out || !slot_row || !out) return MOE_ERR_NULL;
  if ((v = check_align({{slot_out, 16}, {slot_row, 4}, {out, 16}}))) return v;
  if ((v = check_device())) return v;
  return status_of(launch_combine(resolve(p), slot_out, slot_row, out, (hipStream_t)stream));
}

int moe_forward(const moe_problem* p, const void* x, const int32_t* topk_ids,
                const float* topk_weights, const void* w13, const float* w13_scales,
                const void* w2, const float* w2_scales, void* out, void* workspace,
                size_t workspace_bytes, void* stream) {
  int v = validate(p);
  if (v) return v;
  if (is_mx(p)) return MOE_ERR_DTYPE;
  if (!x || !topk_ids || !topk_weights || !w13 || !w2 || !out || !workspace) return MOE_ERR_NULL;
  const bool fp8 = p->w_dtype == MOE_E4M3;
  if (fp8 && (!w13_scales || !w2_scales)) return MOE_ERR_NULL;
  const Resolved r = resolve(p);
  const Layout L = layout(r);
  if ((int64_t)workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  if ((v = check_align({{x, 16}, {topk_ids, 4}, {topk_weights, 4}, {w13, 16}, {w13_scales, 4},
                        {w2, 16}, {w2_scales, 4}, {out, 16}, {workspace, 256}})))
    return v;
  if ((v = check_device())) return v;
  return forward_in(r, L, (char*)workspace, nullptr, x, topk_ids, topk_weights, w13, w13_scales,
                    w2, w2_scales, out, (hipStream_t)stream);
}

int moe_forward_scratch(const moe_problem* p, const void* x, const int32_t* topk_ids,
                        const float* topk_weights, const void* w13, const float* w13_scales,
                        const void* w2, const float* w2_scales, void* out, int32_t* n_invalid,
                        void* stream) {
  int v = validate(p);
  if (v) return v;
  if (is_mx(p)) return MOE_ERR_DTYPE;
  if (!x || !topk_ids || !topk_weights || !w13 || !w2 || !out) return MOE_ERR_NULL;
  const bool fp8 = p->w_dtype == MOE_E4M3;
  if (fp8 && (!w13_scales || !w2_scales)) return MOE_ERR_NULL;
  const Resolved r = resolve(p);
  const Layout L = layout(r);
  if (L.total > (int64_t)MOE_SCRATCH_MAX_BYTES) return MOE_ERR_WORKSPACE;
  if ((v = check_align({{x, 16}, {topk_ids, 4}, {topk_weights, 4}, {w13, 16}, {w13_scales, 4},
                        {w2, 16}, {w2_scales, 4}, {out, 16}, {n_invalid, 4}})))
    return v;
  if ((v = check_device())) return v;
  char* ws = scratch_ptr();
  if (!ws) return MOE_ERR_DEVICE;
  return forward_in(r, L, ws, n_invalid, x, topk_ids, topk_weights, w13, w13_scales, w2,
                    w2_scales, out, (hipStream_t)stream);
}

int64_t moe_scratch_max_bytes(void) { return (int64_t)MOE_SCRATCH_MAX_BYTES; }

}  // extern "C"
