// C ABI of the MoE-VQ routed-expert library: argument validation, workspace layout
// and kernel launches.  Every check runs on the host before any HIP call; the
// library allocates nothing and keeps no per-call state.
#include <string.h>

#include <mutex>

#include "moe_vq_internal.h"
#include "moe_vq_launch.h"

using namespace mvq;

namespace {

thread_local hipError_t g_last_hip_error = hipSuccess;

// Record a failed HIP call and map it to MOE_VQ_EHIP.
int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_VQ_OK;
  g_last_hip_error = e;
  return MOE_VQ_EHIP;
}

bool dims_ok(int H, int I, int E, int k) {
  if (H < 128 || H > MAX_DIM || H % 128) return false;
  if (I < 128 || I > MAX_DIM || I % 128) return false;
  if (E < 1 || E > MAX_E) return false;
  if (k < 1 || k > MAX_K || k > E) return false;
  return true;
}

int check_layer(const moe_vq_layer* L) {
  if (!L) return MOE_VQ_EINVAL;
  if (!dims_ok(L->hidden, L->inter, L->n_experts, L->top_k)) return MOE_VQ_EINVAL;
  if (!L->router_w || !L->codebook || !L->pool || !L->slots) return MOE_VQ_EINVAL;
  if (((uintptr_t)L->pool & 255) || ((uintptr_t)L->codebook & 7) || ((uintptr_t)L->router_w & 15) ||
      ((uintptr_t)L->slots & 7))
    return MOE_VQ_EINVAL;
  if (L->pool_bytes == 0) return MOE_VQ_EINVAL;
  if (!(L->swiglu_limit >= 0.f && L->swiglu_limit <= 3.4e38f)) return MOE_VQ_EINVAL;  // finite, >= 0 (NaN fails)
  if (L->delta_slots) {  // FP4 delta cache: copies listed as experts E + e
    if (2 * L->n_experts > MAX_E || ((uintptr_t)L->delta_slots & 7)) return MOE_VQ_EINVAL;
    if (!(L->gate_tau >= 0.f && L->gate_tau <= 3.4e38f)) return MOE_VQ_EINVAL;
  }
  return MOE_VQ_OK;
}

// Experts the worklist can list: E, or 2E with an FP4 delta cache (the copy of e is E + e).
int virt_experts(const moe_vq_layer* L) { return L->delta_slots ? 2 * L->n_experts : L->n_experts; }

WsLayout layout_of(const moe_vq_layer* L, int T) {
  return ws_layout(L->n_experts, L->hidden, L->inter, L->top_k, T, virt_experts(L));
}

uint32_t key_of(const moe_vq_layer* L, int T) {
  return shape_key(T, virt_experts(L), L->top_k, L->hidden, L->inter);
}

int check_ws(const moe_vq_layer* L, int T, const void* ws, size_t ws_bytes) {
  if (!ws || ((uintptr_t)ws & 255)) return MOE_VQ_EINVAL;
  const WsLayout W = layout_of(L, T);
  if (ws_bytes < W.total) return MOE_VQ_ENOSPACE;
  return MOE_VQ_OK;
}

// Compute units of the current device, queried once per device (idempotent cache).
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  if (dev >= 0 && dev < 64) cached[dev] = n;
  return n;
}


template <typename T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }

FcArgs make_fc_args(const moe_vq_layer* L, int T, void* ws, const WsLayout& W, bool fc1) {
  FcArgs a{};
  a.pool = L->pool;
  a.codebook = static_cast<const uint16_t*>(L->codebook);
  a.hdr = at<uint32_t>(ws, W.hdr);
  a.act_start = at<const int32_t>(ws, W.act_start);
  a.act_off = at<const uint64_t>(ws, W.act_off);
  a.act_fmt = at<const uint32_t>(ws, W.act_fmt);
  a.grp = at<const int32_t>(ws, fc1 ? W.grp1 : W.grp2);
  a.rec = at<const GroupRec>(ws, fc1 ? W.rec1 : W.rec2);
  a.pair_list = at<const int32_t>(ws, W.pair_list);
  a.pair_w = at<const float>(ws, W.pair_w);
  a.x_h = at<const uint16_t>(ws, W.x_h);
  a.x_sc = at<const float>(ws, W.x_sc);
  a.T = T;
  a.H = L->hidden;
  a.I = L->inter;
  a.k = L->top_k;
  a.KS = W.KS;
  a.E = virt_experts(L);
  a.key = key_of(L, T);
  a.lim = L->swiglu_limit;
  a.vq2 = slot_layout(MOE_VQ_FMT_VQ2, L->hidden, L->inter);
  a.mx4 = slot_layout(MOE_VQ_FMT_MXFP4, L->hidden, L->inter);
  return a;
}

// Kernel arguments of the routing launches.
void route_args(const moe_vq_layer* L, const void* x, int x_dtype, int T, int32_t* topk_ids, float* topk_w, void* ws,
                RouteArgs& ra, WorklistArgs& wa) {
  const int E = L->n_experts, H = L->hidden, I = L->inter, k = L->top_k;
  const WsLayout W = layout_of(L, T);
  ra = RouteArgs{};
  ra.router_w = static_cast<const uint16_t*>(L->router_w);
  ra.x = x;
  ra.T = T; ra.H = H; ra.E = E; ra.k = k; ra.KS = W.KS;
  ra.ksp = (W.KS + 3) & ~3;
  ra.logits = at<float>(ws, W.logits);
  ra.x_h = at<uint16_t>(ws, W.x_h);
  ra.x_sc = at<float>(ws, W.x_sc);
  ra.topk_ids = topk_ids;
  ra.topk_w = topk_w;
  ra.pair_w = at<float>(ws, W.pair_w);
  wa = WorklistArgs{};
  wa.x = x;
  wa.x_dtype = x_dtype;
  wa.topk_ids = topk_ids;
  wa.slots = L->slots;
  wa.delta_slots = L->delta_slots;
  wa.pair_w = at<const float>(ws, W.pair_w);
  wa.tau = L->gate_tau;
  wa.pool_bytes = L->pool_bytes;
  wa.T = T; wa.E = E; wa.k = k; wa.H = H; wa.I = I;
  wa.EV = virt_experts(L);
  wa.MT1 = W.MT1;
  wa.MT2 = W.MT2;
  wa.rec1 = at<GroupRec>(ws, W.rec1);
  wa.rec2 = at<GroupRec>(ws, W.rec2);
  wa.G1 = W.G1;
  wa.G2 = W.G2;
  wa.hdr = at<uint32_t>(ws, W.hdr);
  wa.act_expert = at<int32_t>(ws, W.act_expert);
  wa.act_start = at<int32_t>(ws, W.act_start);
  wa.act_off = at<uint64_t>(ws, W.act_off);
  wa.act_fmt = at<uint32_t>(ws, W.act_fmt);
  wa.grp1 = at<int32_t>(ws, W.grp1);
  wa.grp2 = at<int32_t>(ws, W.grp2);
  wa.pair_list = at<int32_t>(ws, W.pair_list);
  wa.key = key_of(L, T);
  // the matrix-core FC launches' grids, for the worklist's split of their tiles by cost
  // (the FC launches compute the same grids; a kernel checks it before using the split)
  wa.part1 = at<int32_t>(ws, W.part1);
  wa.part2 = at<int32_t>(ws, W.part2);
  const int n_cu = device_cu_count();
  if (W.MT1 == MF_MT && mf_supported(H, true)) {
    const int rows = mf_tile_rows(H / 1024, true);
    wa.rb1 = (I + rows - 1) / rows;
    wa.grid1 = mf_grid(n_cu, W.G1, I, rows);
  }
  if (W.MT2 == MF_MT && mf_supported(I, false)) {
    const int rows = mf_tile_rows(I / 1024, false);
    wa.rb2 = (H + rows - 1) / rows;
    wa.grid2 = mf_grid(n_cu, W.G2, H, rows);
  }
  if (wa.grid1 > MAX_PART) wa.grid1 = 0;
  if (wa.grid2 > MAX_PART) wa.grid2 = 0;
}

// The launches of one call, after its arguments have been checked.
hipError_t route_on(const moe_vq_layer* L, const void* x, int x_dtype, int T, int32_t* topk_ids, float* topk_w,
                    void* ws, hipStream_t stream) {
  RouteArgs ra;
  WorklistArgs wa;
  route_args(L, x, x_dtype, T, topk_ids, topk_w, ws, ra, wa);
  return launch_route(ra, x_dtype, wa, stream);
}

hipError_t fc1_on(const moe_vq_layer* L, const void* x, int x_dtype, int T, void* ws, float* h, hipStream_t stream) {
  const WsLayout W = layout_of(L, T);
  FcArgs a = make_fc_args(L, T, ws, W, true);
  a.x_addr = (uint64_t)(uintptr_t)x;
  a.x_dtype = x_dtype;
  a.out = h;
  a.max_groups = W.G1;
  a.part = at<const int32_t>(ws, W.part1);
  return launch_fc1(a, W.MT1, W.G1, device_cu_count(), stream);
}

hipError_t fc2_on(const moe_vq_layer* L, const float* h, int T, void* ws, float* y, hipStream_t stream,
                  bool accumulate = false) {
  const WsLayout W = layout_of(L, T);
  FcArgs a = make_fc_args(L, T, ws, W, false);
  a.h_in = h;
  a.out = at<float>(ws, W.o_buf);
  a.y = y;
  a.accumulate = accumulate ? 1 : 0;
  a.max_groups = W.G2;
  a.part = at<const int32_t>(ws, W.part2);
  return launch_fc2(a, W.MT2, W.G2, device_cu_count(), stream);
}

// Arguments of moe_vq_forward and its static-workspace variant, workspace aside.
int check_forward(const moe_vq_layer* L, const void* x, int x_dtype, int n_tokens, const int32_t* topk_ids,
                  const float* topk_w, const float* h, const float* y) {
  int st = check_layer(L);
  if (st) return st;
  if (n_tokens < 0 || n_tokens > MAX_T) return MOE_VQ_EINVAL;
  if (x_dtype != MOE_VQ_F32 && x_dtype != MOE_VQ_BF16) return MOE_VQ_EINVAL;
  if (n_tokens == 0) return MOE_VQ_OK;
  if (!x || !topk_ids || !topk_w || !h || !y) return MOE_VQ_EINVAL;
  if (((uintptr_t)x & 15) || ((uintptr_t)h & 15) || ((uintptr_t)y & 15)) return MOE_VQ_EINVAL;
  return MOE_VQ_OK;
}

hipError_t forward_on(const moe_vq_layer* L, const void* x, int x_dtype, int T, int32_t* topk_ids, float* topk_w,
                      float* h, float* y, void* ws, hipStream_t stream) {
  hipError_t e = route_on(L, x, x_dtype, T, topk_ids, topk_w, ws, stream);
  if (e == hipSuccess) e = fc1_on(L, x, x_dtype, T, ws, h, stream);
  if (e == hipSuccess) e = fc2_on(L, h, T, ws, y, stream);
  return e;
}

// ---- Workspace of moe_vq_forward_static: one array per GPU, in the library's own device
// memory, held until the process ends.  Host code never uses the array's name as an
// address: its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)16 << 20;
constexpr int MAX_DEVICES = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[STATIC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mutex;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The current device's address of `scratch`, looked up on the device's first call.
hipError_t static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

namespace mvq {
KernelTiming& kernel_timing() {
  thread_local KernelTiming t;
  return t;
}
}  // namespace mvq

extern "C" {

size_t moe_vq_expert_bytes(int format, int hidden, int inter) {
  if (format != MOE_VQ_FMT_VQ2 && format != MOE_VQ_FMT_MXFP4) return 0;
  if (hidden < 128 || hidden > MAX_DIM || hidden % 128 || inter < 128 || inter > MAX_DIM || inter % 128)
    return 0;
  return (size_t)slot_layout(format, hidden, inter).total;
}

int moe_vq_slot_layout(int format, int hidden, int inter, uint64_t offsets[7]) {
  if (!offsets || moe_vq_expert_bytes(format, hidden, inter) == 0) return MOE_VQ_EINVAL;
  const SlotLayout L = slot_layout(format, hidden, inter);
  offsets[0] = L.q_gate; offsets[1] = L.q_up; offsets[2] = L.q_down;
  offsets[3] = L.s_gate; offsets[4] = L.s_up; offsets[5] = L.s_down;
  offsets[6] = L.total;
  return MOE_VQ_OK;
}

size_t moe_vq_workspace_bytes(const moe_vq_layer* L, int n_tokens) {
  if (!L || !dims_ok(L->hidden, L->inter, L->n_experts, L->top_k)) return 0;
  if (n_tokens < 0 || n_tokens > MAX_T) return 0;
  if (L->delta_slots && 2 * L->n_experts > MAX_E) return 0;
  return layout_of(L, n_tokens).total;
}

int moe_vq_route_topk(const moe_vq_layer* L, const void* x, int x_dtype, int n_tokens,
                      int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  int st = check_layer(L);
  if (st) return st;
  if (n_tokens < 0 || n_tokens > MAX_T) return MOE_VQ_EINVAL;
  if (x_dtype != MOE_VQ_F32 && x_dtype != MOE_VQ_BF16) return MOE_VQ_EINVAL;
  if (n_tokens == 0) return MOE_VQ_OK;
  if (!x || !topk_ids || !topk_w || ((uintptr_t)x & 15)) return MOE_VQ_EINVAL;
  if ((st = check_ws(L, n_tokens, ws, ws_bytes))) return st;
  return hip_status(route_on(L, x, x_dtype, n_tokens, topk_ids, topk_w, ws, static_cast<hipStream_t>(stream)));
}

int moe_vq_fc1_silu(const moe_vq_layer* L, const void* x, int x_dtype, int n_tokens, void* ws, size_t ws_bytes,
                    float* h, void* stream) {
  int st = check_layer(L);
  if (st) return st;
  if (n_tokens < 0 || n_tokens > MAX_T) return MOE_VQ_EINVAL;
  if (x_dtype != MOE_VQ_F32 && x_dtype != MOE_VQ_BF16) return MOE_VQ_EINVAL;
  if (n_tokens == 0) return MOE_VQ_OK;
  if (!x || !h || ((uintptr_t)x & 15) || ((uintptr_t)h & 15)) return MOE_VQ_EINVAL;
  if ((st = check_ws(L, n_tokens, ws, ws_bytes))) return st;
  return hip_status(fc1_on(L, x, x_dtype, n_tokens, ws, h, static_cast<hipStream_t>(stream)));
}

int moe_vq_fc2_combine(const moe_vq_layer* L, const float* h, int n_tokens, void* ws, size_t ws_bytes,
                       float* y, void* stream) {
  int st = check_layer(L);
  if (st) return st;
  if (n_tokens < 0 || n_tokens > MAX_T) return MOE_VQ_EINVAL;
  if (n_tokens == 0) return MOE_VQ_OK;
  if (!h || !y || ((uintptr_t)h & 15) || ((uintptr_t)y & 15)) return MOE_VQ_EINVAL;
  if ((st = check_ws(L, n_tokens, ws, ws_bytes))) return st;
  return hip_status(fc2_on(L, h, n_tokens, ws, y, static_cast<hipStream_t>(stream)));
}

int moe_vq_forward(const moe_vq_layer* L, const void* x, int x_dtype, int n_tokens, int32_t* topk_ids,
                   float* topk_w, float* h, float* y, void* ws, size_t ws_bytes, void* stream) {
  int st = check_forward(L, x, x_dtype, n_tokens, topk_ids, topk_w, h, y);
  if (st || n_tokens == 0) return st;
  if ((st = check_ws(L, n_tokens, ws, ws_bytes))) return st;
  return hip_status(forward_on(L, x, x_dtype, n_tokens, topk_ids, topk_w, h, y, ws, static_cast<hipStream_t>(stream)));
}

int moe_vq_forward_static(const moe_vq_layer* L, const void* x, int x_dtype, int n_tokens, int32_t* topk_ids,
                          float* topk_w, float* h, float* y, int32_t* status, void* stream) {
  int st = check_forward(L, x, x_dtype, n_tokens, topk_ids, topk_w, h, y);
  if (st || n_tokens == 0) return st;
  if ((uintptr_t)status & 3) return MOE_VQ_EINVAL;
  if (layout_of(L, n_tokens).total > STATIC_SCRATCH_BYTES)
    return MOE_VQ_ENOSPACE;
  void* ws = nullptr;
  if ((st = hip_status(static_scratch(&ws)))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = hip_status(forward_on(L, x, x_dtype, n_tokens, topk_ids, topk_w, h, y, ws, s)))) return st;
  if (status)  // the status word and the offending expert, for the caller to read
    return hip_status(hipMemcpyAsync(status, ws, 2 * sizeof(int32_t), hipMemcpyDeviceToDevice, s));
  return MOE_VQ_OK;
}

int moe_vq_shared_expert(const moe_vq_layer* L, const void* x, int x_dtype, int n_tokens, void* ws,
                         size_t ws_bytes, float* h, float* y, void* stream) {
  int st = check_layer(L);
  if (st) return st;
  if (L->n_experts != 1 || L->top_k != 1) return MOE_VQ_EINVAL;
  if (n_tokens < 0 || n_tokens > MAX_T) return MOE_VQ_EINVAL;
  if (x_dtype != MOE_VQ_F32 && x_dtype != MOE_VQ_BF16) return MOE_VQ_EINVAL;
  if (n_tokens == 0) return MOE_VQ_OK;
  if (!x || !h || !y || ((uintptr_t)x & 15) || ((uintptr_t)h & 15) || ((uintptr_t)y & 15)) return MOE_VQ_EINVAL;
  if ((st = check_ws(L, n_tokens, ws, ws_bytes))) return st;
  // The one-expert layer's routing (every token to expert 0 with weight 1), FC1 and FC2
  // with the combine adding to y.  The selection goes to the workspace's per-pair
  // arrays' neighbours: routing needs somewhere to write ids and weights, and with k = 1
  // and one expert they carry nothing the caller needs.
  const WsLayout W = layout_of(L, n_tokens);
  int32_t* ids = at<int32_t>(ws, W.o_buf);
  float* w = at<float>(ws, W.o_buf + (size_t)n_tokens * 4);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = route_on(L, x, x_dtype, n_tokens, ids, w, ws, s);
  if (e == hipSuccess) e = fc1_on(L, x, x_dtype, n_tokens, ws, h, s);
  if (e == hipSuccess) e = fc2_on(L, h, n_tokens, ws, y, s, true);
  return hip_status(e);
}

int moe_vq_prefill_gemm(const moe_vq_layer* L, const void* x, int x_dtype, int n_tokens, void* ws,
                        size_t ws_bytes, float* y, void* stream) {
  int st = check_layer(L);
  if (st) return st;
  if (n_tokens < 0 || n_tokens > MAX_T) return MOE_VQ_EINVAL;
  if (x_dtype != MOE_VQ_F32 && x_dtype != MOE_VQ_BF16) return MOE_VQ_EINVAL;
  if (n_tokens == 0) return MOE_VQ_OK;
  if (!x || !y || ((uintptr_t)x & 15) || ((uintptr_t)y & 15)) return MOE_VQ_EINVAL;
  if ((st = check_ws(L, n_tokens, ws, ws_bytes))) return st;
  const int H = L->hidden, I = L->inter, k = L->top_k, T = n_tokens;
  const WsLayout W = layout_of(L, T);
  PrefillArgs a{};
  a.pool = L->pool;
  a.codebook = static_cast<const uint16_t*>(L->codebook);
  a.hdr = at<uint32_t>(ws, W.hdr);
  a.act_start = at<const int32_t>(ws, W.act_start);
  a.act_off = at<const uint64_t>(ws, W.act_off);
  a.act_fmt = at<const uint32_t>(ws, W.act_fmt);
  a.pair_list = at<const int32_t>(ws, W.pair_list);
  a.pair_w = at<const float>(ws, W.pair_w);
  a.x = x;
  a.x_dtype = x_dtype;
  a.x16 = at<uint16_t>(ws, W.x16);
  a.x16_e = at<int32_t>(ws, W.x16_e);
  a.mt_pre = at<int32_t>(ws, W.mt_pre);
  a.hmax = at<uint32_t>(ws, W.hmax);
  a.h = at<uint16_t>(ws, W.h_pre);
  a.o_buf = at<float>(ws, W.o_buf);
  a.y = y;
  a.T = T; a.H = H; a.I = I; a.k = k; a.E = virt_experts(L);
  a.lim = L->swiglu_limit;
  a.key = key_of(L, T);
  a.vq2 = slot_layout(MOE_VQ_FMT_VQ2, H, I);
  a.mx4 = slot_layout(MOE_VQ_FMT_MXFP4, H, I);
  return hip_status(launch_prefill(a, x_dtype, static_cast<hipStream_t>(stream)));
}

int moe_vq_decode_expert(const moe_vq_layer* L, int expert, int matrix, int out_dtype, void* out,
                         int32_t* status_dev, void* stream) {
  int st = check_layer(L);
  if (st) return st;
  if (expert < 0 || expert >= L->n_experts) return MOE_VQ_EINVAL;
  if (matrix < MOE_VQ_MAT_GATE || matrix > MOE_VQ_MAT_DOWN) return MOE_VQ_EINVAL;
  if (out_dtype != MOE_VQ_F32 && out_dtype != MOE_VQ_BF16) return MOE_VQ_EINVAL;
  if (!out || ((uintptr_t)out & 15)) return MOE_VQ_EINVAL;
  return hip_status(launch_decode_expert(L->pool, L->slots, L->pool_bytes,
                                         static_cast<const uint16_t*>(L->codebook), L->hidden, L->inter,
                                         expert, matrix, out_dtype, out, status_dev,
                                         static_cast<hipStream_t>(stream)));
}

int moe_vq_check(const void* ws, void* stream, int32_t* info) {
  if (!ws) return MOE_VQ_EINVAL;
  uint32_t hdr[2] = {0, 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st = hip_status(hipStreamSynchronize(s));
  if (st) return st;
  if ((st = hip_status(hipMemcpy(hdr, ws, sizeof(hdr), hipMemcpyDeviceToHost)))) return st;
  if (info) *info = (int32_t)hdr[1];
  return (int)hdr[0];
}

// The step's header and distinct experts (adjacent in the workspace) in one
// stream-ordered copy.  With a pinned staging buffer of HDR_WORDS + E words the copy is
// asynchronous and one stream synchronisation covers it; without one it goes through a
// host array on the stack, which HIP copies synchronously.
static int read_step(const moe_vq_layer* L, int n_tokens, const void* ws, int32_t summary[4], int32_t* experts,
                     void* stream, uint32_t* pinned) {
  if (!L || !dims_ok(L->hidden, L->inter, L->n_experts, L->top_k)) return MOE_VQ_EINVAL;
  if (!ws || !summary || n_tokens < 0 || n_tokens > MAX_T) return MOE_VQ_EINVAL;
  if (L->delta_slots && 2 * L->n_experts > MAX_E) return MOE_VQ_EINVAL;
  const int E = virt_experts(L);  // (the listed experts include the FP4 copies, E + e)
  const WsLayout W = layout_of(L, n_tokens);
  static_assert(HDR_WORDS * 4 % 256 == 0, "the expert list must follow the header");
  uint32_t local[HDR_WORDS + MAX_E];
  uint32_t* buf = pinned ? pinned : local;
  const size_t words = experts ? HDR_WORDS + (size_t)E : HDR_WORDS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st = hip_status(hipMemcpyAsync(buf, static_cast<const char*>(ws) + W.hdr, words * 4, hipMemcpyDeviceToHost, s));
  if (st) return st;
  if ((st = hip_status(hipStreamSynchronize(s)))) return st;
  summary[0] = (int32_t)buf[HDR_STATUS];
  summary[1] = (int32_t)buf[HDR_INFO];
  summary[2] = (int32_t)buf[HDR_N_ACTIVE];
  summary[3] = (int32_t)buf[HDR_N_PAIRS];
  if (experts && buf[HDR_N_ACTIVE] > 0) {
    const size_t n = buf[HDR_N_ACTIVE] <= (uint32_t)E ? buf[HDR_N_ACTIVE] : (size_t)E;
    memcpy(experts, buf + HDR_WORDS, n * 4);
  }
  return MOE_VQ_OK;
}

int moe_vq_step_info(const moe_vq_layer* L, int n_tokens, const void* ws, int32_t summary[4],
                     int32_t* experts, void* stream) {
  return read_step(L, n_tokens, ws, summary, experts, stream, nullptr);
}

// ---- Host-RAM expert tier (see moe_vq.h) ----------------------------------------------

int moe_vq_tier_plan(const moe_vq_tier* tier, int n_experts, const int32_t* active, int n_active,
                     int32_t* install_expert, int32_t* install_slot, int32_t* evict_expert, int* n_install) {
  if (!tier || !n_install || n_experts < 1 || n_experts > MAX_E || n_active < 0 || n_active > n_experts)
    return MOE_VQ_EINVAL;
  if (n_active > 0 && (!active || !install_expert || !install_slot || !evict_expert)) return MOE_VQ_EINVAL;
  const int ns = tier->n_dev_slots;
  if (ns < 1 || ns > 4096 || !tier->host_slots || !tier->dev_slot_expert || !tier->dev_slot_stamp)
    return MOE_VQ_EINVAL;
  *n_install = 0;
  // slots held by an active expert are not candidates; an expert is resident if a slot
  // holds it
  bool is_active[MAX_E] = {};
  for (int i = 0; i < n_active; ++i) {
    if (active[i] < 0 || active[i] >= n_experts) return MOE_VQ_EINVAL;
    is_active[active[i]] = true;
  }
  int slot_of[MAX_E];
  for (int e = 0; e < n_experts; ++e) slot_of[e] = -1;
  for (int s = 0; s < ns; ++s) {
    const int e = tier->dev_slot_expert[s];
    if (e >= n_experts) return MOE_VQ_EINVAL;
    if (e >= 0) slot_of[e] = s;
  }
  bool taken[4096] = {};  // slots assigned by this plan
  int n = 0;
  for (int i = 0; i < n_active; ++i) {
    const int e = active[i];
    if (slot_of[e] >= 0) continue;
    const uint32_t f = tier->host_slots[e].format;
    if (f != MOE_VQ_FMT_VQ2 && f != MOE_VQ_FMT_MXFP4) continue;  // not in the host pool either
    int best = -1;
    for (int s = 0; s < ns && best < 0; ++s)
      if (!taken[s] && tier->dev_slot_expert[s] < 0) best = s;
    if (best < 0) {
      for (int s = 0; s < ns; ++s) {
        const int h = tier->dev_slot_expert[s];
        if (taken[s] || h < 0 || is_active[h]) continue;
        if (best < 0 || tier->dev_slot_stamp[s] < tier->dev_slot_stamp[best]) best = s;
      }
    }
    if (best < 0) { *n_install = 0; return MOE_VQ_ENOSPACE; }
    taken[best] = true;
    install_expert[n] = e;
    install_slot[n] = best;
    evict_expert[n] = tier->dev_slot_expert[best];
    ++n;
  }
  *n_install = n;
  return MOE_VQ_OK;
}

int moe_vq_tier_init(const moe_vq_layer* L, moe_vq_tier* tier, moe_vq_slot* slots, void* stream) {
  if (!L || !dims_ok(L->hidden, L->inter, L->n_experts, L->top_k) || !tier || !slots) return MOE_VQ_EINVAL;
  const int ns = tier->n_dev_slots, E = L->n_experts;
  if (ns < 1 || ns > 4096 || !tier->host_pool || !tier->host_slots || !tier->dev_slot_offsets ||
      !tier->dev_slot_expert || !tier->dev_slot_stamp || !tier->slot_mirror)
    return MOE_VQ_EINVAL;
  const size_t need = moe_vq_expert_bytes(MOE_VQ_FMT_MXFP4, L->hidden, L->inter) >
                              moe_vq_expert_bytes(MOE_VQ_FMT_VQ2, L->hidden, L->inter)
                          ? moe_vq_expert_bytes(MOE_VQ_FMT_MXFP4, L->hidden, L->inter)
                          : moe_vq_expert_bytes(MOE_VQ_FMT_VQ2, L->hidden, L->inter);
  for (int s = 0; s < ns; ++s) {
    const uint64_t o = tier->dev_slot_offsets[s];
    if ((o & 255) || o > L->pool_bytes || need > L->pool_bytes - o) return MOE_VQ_EINVAL;
  }
  for (int s = 0; s < ns; ++s) { tier->dev_slot_expert[s] = -1; tier->dev_slot_stamp[s] = 0; }
  for (int e = 0; e < E; ++e) tier->slot_mirror[e] = moe_vq_slot{0, MOE_VQ_FMT_ABSENT, 0};
  tier->step = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int r = hip_status(hipMemcpyAsync(slots, tier->slot_mirror, (size_t)E * sizeof(moe_vq_slot),
                                    hipMemcpyHostToDevice, st));
  if (r) return r;
  return hip_status(hipStreamSynchronize(st));
}

int moe_vq_tier_resolve(const moe_vq_layer* L, moe_vq_tier* tier, uint8_t* pool, moe_vq_slot* slots,
                        int n_tokens, const void* ws, void* stream, int32_t* n_installed) {
  if (n_installed) *n_installed = 0;
  if (!L || !dims_ok(L->hidden, L->inter, L->n_experts, L->top_k) || !tier || !pool || !slots || !ws)
    return MOE_VQ_EINVAL;
  if (n_tokens < 0 || n_tokens > MAX_T || !tier->slot_mirror || !tier->dev_slot_offsets || !tier->host_pool)
    return MOE_VQ_EINVAL;
  const int E = L->n_experts, EV = virt_experts(L);
  int32_t summary[4];
  int32_t active[MAX_E];
  // (the pinned read-back buffer has room for E listed experts: with an FP4 delta cache,
  // which can list 2E, the read goes through the stack instead)
  int r = read_step(L, n_tokens, ws, summary, active, stream,
                    EV == E ? tier->readback : nullptr);  // (synchronises stream)
  if (r) return r;
  const int n_listed = summary[2] < 0 ? 0 : (summary[2] > EV ? EV : summary[2]);
  int n_active = 0;  // the tier manages slots[] only: FP4 copies (E + e) are left out
  for (int i = 0; i < n_listed; ++i)
    if (active[i] >= 0 && active[i] < E) active[n_active++] = active[i];
  tier->step += 1;
  for (int s = 0; s < tier->n_dev_slots; ++s) {
    const int e = tier->dev_slot_expert[s];
    if (e < 0) continue;
    for (int i = 0; i < n_active; ++i)
      if (active[i] == e) { tier->dev_slot_stamp[s] = tier->step; break; }
  }
  int32_t ie[MAX_E], is[MAX_E], ev[MAX_E];
  int n = 0;
  if ((r = moe_vq_tier_plan(tier, E, active, n_active, ie, is, ev, &n))) return r;
  if (n == 0) return MOE_VQ_OK;  // nothing enqueued since the synchronisation above
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int i = 0; i < n; ++i) {
    const int e = ie[i], sl = is[i];
    const moe_vq_slot hs = tier->host_slots[e];
    const size_t bytes = moe_vq_expert_bytes((int)hs.format, L->hidden, L->inter);
    const uint64_t dst = tier->dev_slot_offsets[sl];
    if ((r = hip_status(hipMemcpyAsync(pool + dst, tier->host_pool + hs.byte_offset, bytes,
                                       hipMemcpyHostToDevice, st))))
      return r;
    if (ev[i] >= 0) tier->slot_mirror[ev[i]] = moe_vq_slot{0, MOE_VQ_FMT_ABSENT, 0};
    tier->slot_mirror[e] = moe_vq_slot{dst, hs.format, 0};
    tier->dev_slot_expert[sl] = e;
    tier->dev_slot_stamp[sl] = tier->step;
    if (n_installed) *n_installed = i + 1;
  }
  if ((r = hip_status(hipMemcpyAsync(slots, tier->slot_mirror, (size_t)E * sizeof(moe_vq_slot),
                                     hipMemcpyHostToDevice, st))))
    return r;
  return hip_status(hipStreamSynchronize(st));
}

int moe_vq_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || ((uintptr_t)buf & 15) || ((uintptr_t)sink & 3) || bytes < 16 || (bytes & 15))
    return MOE_VQ_EINVAL;
  return hip_status(launch_read_probe(buf, bytes, sink, device_cu_count(), static_cast<hipStream_t>(stream)));
}

int moe_vq_time_next_kernel(void* start_event, void* stop_event) {
  kernel_timing() = KernelTiming{static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  return MOE_VQ_OK;
}

const char* moe_vq_last_hip_error(void) {
  return g_last_hip_error == hipSuccess ? "" : hipGetErrorString(g_last_hip_error);
}

const char* moe_vq_strerror(int status) {
  switch (status) {
    case MOE_VQ_OK: return "ok";
    case MOE_VQ_EINVAL: return "invalid argument";
    case MOE_VQ_EUNSUPPORTED: return "unsupported shape or dtype";
    case MOE_VQ_ENOSPACE: return "workspace too small";
    case MOE_VQ_EHIP: return "HIP runtime error";
    case MOE_VQ_ENOTRESIDENT: return "selected expert not resident in the slot pool";
    default: return "unknown status";
  }
}

}  // extern "C"
