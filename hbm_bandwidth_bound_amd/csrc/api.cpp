// api.cpp -- host side of the C ABI declared in include/kie.h: validation, set-up, launches.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/kie.h"
#include "../../include/kie_measure.h"
#include "layout.h"
#include "monokernel.h"
#include "prefill.h"

namespace kie {
hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, int32_t blocks, hipStream_t st);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks, hipStream_t st);
}  // namespace kie

using namespace kie;

static const int64_t kDefaultTimeoutTicks = 200000000;  // 2 s per wait (s_memrealtime runs at 100 MHz)

struct kie_ctx {
  Shape s;
  Exch exo;
  Workspace wso;
  int device;
  hipStream_t stream;
  uint8_t* packed;
  uint16_t* kv;
  uint8_t* ws;
  KernelFn kernel;
  KernelFn prompt_kernel;
  int32_t lds;
  bool w8;                 // 8-bit (e4m3fn) layer matrices and LM head
  int32_t pos;
  uint32_t epoch;  // tag of the next step
  bool bad_state;
  int32_t* tok_ring;       // device view of the caller's host ring, or null
  int32_t ring_cap;
  int64_t ring_count;      // tokens streamed to it so far
  int64_t timeout_ticks;
  uint32_t skew;           // kie_set_skew
  int32_t* abort_dev;      // device view of the caller's host abort word, or null
  std::vector<float> wscale_host;  // 8-bit weights: the matrix scales, copied from the caller
  bool static_ws;          // the workspace is this GPU's static array (kie_create_static)
  std::string last_error;
};

static std::string g_create_error;

static void set_err(std::string* dst, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (dst) *dst = buf;
}

#define HIP_TRY(dst, call)                                                               \
  do {                                                                                   \
    hipError_t e_ = (call);                                                              \
    if (e_ != hipSuccess) {                                                              \
      set_err(dst, "%s failed: %s", #call, hipGetErrorString(e_));                       \
      return KIE_ERR_HIP;                                                                \
    }                                                                                    \
  } while (0)

static int query_cus(int* out, std::string* err) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    set_err(err, "no HIP device");
    return KIE_ERR_HIP;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    set_err(err, "cannot query the compute-unit count");
    return KIE_ERR_HIP;
  }
  *out = n;
  return KIE_OK;
}

// Packed-image geometry in the config's weight format (tiles of kTileK bf16 or 2 * kTileK 8-bit
// weights per row).
static bool cfg_w8(const kie_config* c) { return c && c->weight_format == KIE_WEIGHTS_FP8_E4M3; }
static int64_t pk_embed_offset(const Shape& s, bool w8) {
  return w8 ? packed_embed_offset<2 * kTileK>(s) : packed_embed_offset(s);
}
static int64_t pk_bytes(const Shape& s, bool w8) { return w8 ? packed_bytes<2 * kTileK>(s) : packed_bytes(s); }

// Shape from a config; nwg = compute units of the current device (or `nwg_override` > 0).
static kie_status make_shape(const kie_config* c, int nwg_override, Shape* s, std::string* err) {
  if (!c) {
    set_err(err, "config is NULL");
    return KIE_ERR_INVALID_ARG;
  }
  int nwg = nwg_override;
  if (nwg <= 0) {
    kie_status st = query_cus(&nwg, err);
    if (st != KIE_OK) return st;
  }
  s->L = c->n_layers;
  s->d = c->d_model;
  s->nq = c->n_heads;
  s->nkv = c->n_kv_heads;
  s->hd = c->head_dim;
  s->F = c->ffn_dim;
  s->V = c->vocab_size;
  s->max_seq = c->max_seq_len;
  s->eps = c->rms_eps;
  s->theta = c->rope_theta;
  s->nwg = nwg;
  s->E = 0;
  s->A = 0;
  s->Fe = 0;
  const bool moe = c->n_experts != 0;
  if (c->n_layers <= 0 || c->d_model <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      (moe ? c->ffn_dim != 0 : c->ffn_dim <= 0) || c->vocab_size <= 0 || c->max_seq_len <= 0 ||
      !(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) {
    set_err(err, "config has a non-positive size (or a mixture-of-experts config with ffn_dim != 0)");
    return KIE_ERR_INVALID_ARG;
  }
  if (!moe && (c->n_experts_active != 0 || c->expert_ffn_dim != 0)) {
    set_err(err, "n_experts_active and expert_ffn_dim must be 0 when n_experts is 0");
    return KIE_ERR_INVALID_ARG;
  }
  if (moe) {
    if (c->n_experts < 2 || c->n_experts % 2 || c->n_experts > kThreads || c->n_experts_active < 1 ||
        c->n_experts_active > c->n_experts || c->n_experts_active > kMaxActive || c->expert_ffn_dim <= 0 ||
        c->expert_ffn_dim % kTileK) {
      set_err(err, "mixture of experts: n_experts must be even and in [2, %d], n_experts_active in [1, min(%d, "
              "n_experts)], expert_ffn_dim a positive multiple of %d", kThreads, kMaxActive, kTileK);
      return KIE_ERR_UNSUPPORTED;
    }
    s->E = c->n_experts;
    s->A = c->n_experts_active;
    s->Fe = c->expert_ffn_dim;
    s->F = s->A * s->Fe;  // width of the gathered expert activations
    if (expert_tiles(*s) >= (int64_t)0xffffffff) {  // routed tiles are indexed with 32 bits
      set_err(err, "the experts' weights exceed 4 TiB");
      return KIE_ERR_UNSUPPORTED;
    }
  }
  if (c->weight_format != KIE_WEIGHTS_BF16 && c->weight_format != KIE_WEIGHTS_FP8_E4M3) {
    set_err(err, "unknown weight_format %d", c->weight_format);
    return KIE_ERR_INVALID_ARG;
  }
  const bool w8 = cfg_w8(c);
  if (w8 && moe) {
    set_err(err, "8-bit weights are supported for dense layers only");
    return KIE_ERR_UNSUPPORTED;
  }
  const int tk = w8 ? 2 * kTileK : kTileK;
  if (s->d % tk || s->qdim() % tk || s->F % tk) {
    set_err(err, "d_model (%d), n_heads*head_dim (%d) and ffn_dim (%d) must be multiples of %d", s->d, s->qdim(), s->F,
            tk);
    return KIE_ERR_UNSUPPORTED;
  }
  if (s->hd != 64 && s->hd != 128) {
    set_err(err, "head_dim must be 64 or 128 (got %d)", s->hd);
    return KIE_ERR_UNSUPPORTED;
  }
  if (s->nq % s->nkv) {
    set_err(err, "n_heads (%d) must be a multiple of n_kv_heads (%d)", s->nq, s->nkv);
    return KIE_ERR_UNSUPPORTED;
  }
  const int G = s->nq / s->nkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) {
    set_err(err, "n_heads / n_kv_heads must be 1, 2, 4 or 8 (got %d)", G);
    return KIE_ERR_UNSUPPORTED;
  }
  if (s->V % 2 || s->d % 2) {
    set_err(err, "vocab_size and d_model must be even");
    return KIE_ERR_UNSUPPORTED;
  }
  if (nwg > kMaxWG || nwg % s->nkv) {
    set_err(err, "the compute-unit count (%d) must be a multiple of n_kv_heads (%d) and at most %d", nwg, s->nkv,
            kMaxWG);
    return KIE_ERR_UNSUPPORTED;
  }
  for (int st = ST_QKV; st < ST_COUNT; ++st) {
    const int64_t per_wg = ((int64_t)s->stage_pairs(st) + nwg - 1) / nwg;
    const int32_t kt = s->stage_k(st) / tk;
    const int64_t units = per_wg * (kt / unit_tiles(kt));
    if (units > kMaxUnits) {  // per-unit partial sums of one stage live in LDS
      set_err(err, "a weight matrix needs %lld work units per compute unit (at most %d supported)", (long long)units,
              kMaxUnits);
      return KIE_ERR_UNSUPPORTED;
    }
  }
  if ((int64_t)s->V * s->d >= (int64_t)1 << 40) {
    set_err(err, "embedding too large");
    return KIE_ERR_UNSUPPORTED;
  }
  return KIE_OK;
}

extern "C" {

size_t kie_packed_weight_bytes(const kie_config* cfg) {
  Shape s;
  if (make_shape(cfg, 0, &s, nullptr) != KIE_OK) return 0;
  return (size_t)pk_bytes(s, cfg_w8(cfg));
}

size_t kie_kv_cache_bytes(const kie_config* cfg) {
  Shape s;
  if (make_shape(cfg, 0, &s, nullptr) != KIE_OK) return 0;
  return (size_t)kv_bytes(s);
}

size_t kie_workspace_bytes(const kie_config* cfg) {
  Shape s;
  if (make_shape(cfg, 0, &s, nullptr) != KIE_OK) return 0;
  return (size_t)workspace_layout(s).end;
}

int32_t kie_num_workgroups(void) {
  int n = 0;
  kie_status st = query_cus(&n, nullptr);
  return st == KIE_OK ? n : st;
}

const char* kie_status_string(kie_status status) {
  switch (status) {
    case KIE_OK: return "ok";
    case KIE_ERR_INVALID_ARG: return "invalid argument";
    case KIE_ERR_UNSUPPORTED: return "unsupported configuration or device";
    case KIE_ERR_CAPACITY: return "KV capacity exceeded";
    case KIE_ERR_HIP: return "HIP runtime error";
    case KIE_ERR_STATE: return "context holds a device error (call kie_reset)";
    case KIE_ERR_TIMEOUT: return "device wait timed out";
    case KIE_ERR_ABORTED: return "device run aborted";
    default: return "unknown status";
  }
}

const char* kie_last_error(const kie_ctx* ctx) { return ctx ? ctx->last_error.c_str() : g_create_error.c_str(); }

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool aligned256(const void* p) { return ((uintptr_t)p & 255u) == 0; }

// ------------------------------------------------------------------ the static workspace
// For callers that cannot allocate device memory: the workspace of contexts made by
// kie_create_static lives in this array, one copy per GPU (the HIP runtime places it in each
// device's memory when the library's code is loaded there; it stays until the process ends).
// Host code uses only the device address hipGetSymbolAddress returns for the current device,
// never the array's name, which on the host is a stand-in and not a device address.
static __device__ __align__(256) uint8_t scratch[KIE_STATIC_WORKSPACE_MAX];
constexpr int kMaxDevices = 64;
static std::mutex g_static_mu;
static uint8_t* g_static_addr[kMaxDevices];          // device address of `scratch`, once looked up
static const kie_ctx* g_static_owner[kMaxDevices];   // the static context now using it

// Device address of this GPU's `scratch` (the current device), looked up once per device.
static kie_status static_workspace(int dev, uint8_t** addr, std::string* err) {
  if (dev < 0 || dev >= kMaxDevices) {
    set_err(err, "device %d is beyond the %d devices the static workspace supports", dev, kMaxDevices);
    return KIE_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (!g_static_addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      set_err(err, "hipGetSymbolAddress of the static workspace failed: %s", hipGetErrorString(e));
      return KIE_ERR_HIP;
    }
    g_static_addr[dev] = (uint8_t*)p;
  }
  *addr = g_static_addr[dev];
  return KIE_OK;
}
// A static context may enqueue work only while it is the one that last took over the array.
static bool static_owner_ok(const kie_ctx* ctx) {
  if (!ctx->static_ws) return true;
  std::lock_guard<std::mutex> lk(g_static_mu);
  return g_static_owner[ctx->device] == ctx;
}

// kie_create and kie_create_static: workspace == NULL selects this GPU's static array.
static kie_status create_impl(const kie_config* cfg, const kie_weights* src, void* packed, void* kv_cache,
                              void* workspace, void* hip_stream, kie_ctx** out) {
  if (out) *out = nullptr;
  g_create_error.clear();
  std::string* err = &g_create_error;
  const bool static_ws = workspace == nullptr;
  if (!out || !src || !packed || !kv_cache) {
    set_err(err, "NULL argument");
    return KIE_ERR_INVALID_ARG;
  }
  // Checked before anything touches the device. The KV cache and the workspace start on a
  // 256-byte boundary, so that every cache row (128 or 256 bytes) and every workspace piece owns
  // whole cache lines: a row appended by one workgroup is never in a line another workgroup
  // read earlier in the same launch.
  if (!aligned16(packed) || !aligned256(kv_cache) || (!static_ws && !aligned256(workspace))) {
    set_err(err, "packed must be 16-byte aligned, kv_cache and workspace 256-byte aligned");
    return KIE_ERR_INVALID_ARG;
  }
  Shape s;
  kie_status st = make_shape(cfg, 0, &s, err);
  if (st != KIE_OK) return st;
  const int L = s.L;
  const bool moe = s.moe();
  const bool w8 = cfg_w8(cfg);
  if (w8) {
    if (!src->weight_scales) {
      set_err(err, "8-bit weights need weight_scales");
      return KIE_ERR_INVALID_ARG;
    }
    for (int i = 0; i < L * 7 + 1; ++i)
      if (!(fabsf(src->weight_scales[i]) < INFINITY)) {
        set_err(err, "weight_scales[%d] is not finite", i);
        return KIE_ERR_INVALID_ARG;
      }
  }
  if (!src->embed || !src->final_norm || !src->lm_head || !src->attn_norm || !src->wq || !src->wk || !src->wv ||
      !src->wo || !src->ffn_norm ||
      (moe ? (!src->w_router || !src->moe_gate || !src->moe_up || !src->moe_down)
           : (!src->w_gate || !src->w_up || !src->w_down))) {
    set_err(err, "a weight pointer is NULL");
    return KIE_ERR_INVALID_ARG;
  }
  for (int l = 0; l < L; ++l) {
    std::vector<const void*> ps = {src->attn_norm[l], src->wq[l], src->wk[l], src->wv[l], src->wo[l],
                                   src->ffn_norm[l]};
    if (moe)
      ps.insert(ps.end(), {src->w_router[l], src->moe_gate[l], src->moe_up[l], src->moe_down[l]});
    else
      ps.insert(ps.end(), {src->w_gate[l], src->w_up[l], src->w_down[l]});
    for (const void* p : ps) {
      if (!p || !aligned16(p)) {
        set_err(err, "layer %d: a weight pointer is NULL or not 16-byte aligned", l);
        return KIE_ERR_INVALID_ARG;
      }
    }
  }
  if (!aligned16(src->embed) || !aligned16(src->lm_head)) {
    set_err(err, "embed and lm_head must be 16-byte aligned");
    return KIE_ERR_INVALID_ARG;
  }
  int dev = 0;
  HIP_TRY(err, hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIP_TRY(err, hipGetDeviceProperties(&prop, dev));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    set_err(err, "device %s is not gfx950", prop.gcnArchName);
    return KIE_ERR_UNSUPPORTED;
  }
  if (!prop.cooperativeLaunch) {
    set_err(err, "device does not support cooperative launches");
    return KIE_ERR_UNSUPPORTED;
  }
  const int lds_limit = (int)prop.sharedMemPerBlock;
  const int32_t lds = lds_bytes_for(s);
  if (lds > lds_limit) {
    set_err(err, "shape needs %d bytes of LDS per workgroup (device limit %d)", lds, lds_limit);
    return KIE_ERR_UNSUPPORTED;
  }
  KernelFn kfn = decode_kernel_for(s.group(), s.hd, false, moe, w8);
  KernelFn pfn = decode_kernel_for(s.group(), s.hd, true, moe, w8);
  if (!kfn || !pfn) {
    set_err(err, "no kernel for group %d head_dim %d%s", s.group(), s.hd,
            moe ? " with mixture-of-experts layers" : (w8 ? " with 8-bit weights" : ""));
    return KIE_ERR_UNSUPPORTED;
  }
  HIP_TRY(err, hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, lds));
  HIP_TRY(err, hipFuncSetAttribute((const void*)pfn, hipFuncAttributeMaxDynamicSharedMemorySize, lds));
  int occ = 0;
  HIP_TRY(err, hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)kfn, kThreads, lds));
  if (occ < 1) {
    set_err(err, "the decode kernel cannot be resident (occupancy %d)", occ);
    return KIE_ERR_UNSUPPORTED;
  }

  const Workspace wso = workspace_layout(s, !static_ws);
  if (static_ws) {
    if (wso.end > (int64_t)KIE_STATIC_WORKSPACE_MAX) {
      set_err(err, "this configuration needs a %lld-byte workspace; the static workspace holds %llu bytes",
              (long long)wso.end, (unsigned long long)KIE_STATIC_WORKSPACE_MAX);
      return KIE_ERR_CAPACITY;
    }
    uint8_t* ws = nullptr;
    HIP_TRY(err, hipSetDevice(dev));
    st = static_workspace(dev, &ws, err);
    if (st != KIE_OK) return st;
    workspace = ws;
  }

  kie_ctx* c = new kie_ctx();
  c->s = s;
  c->exo = exch_layout(s);
  c->wso = wso;
  c->static_ws = static_ws;
  c->device = dev;
  c->stream = (hipStream_t)hip_stream;
  c->packed = (uint8_t*)packed;
  c->kv = (uint16_t*)kv_cache;
  c->ws = (uint8_t*)workspace;
  c->kernel = kfn;
  c->prompt_kernel = pfn;
  c->lds = lds;
  c->w8 = w8;
  c->pos = 0;
  c->epoch = 1;
  c->bad_state = false;
  c->tok_ring = nullptr;
  c->ring_cap = 0;
  c->ring_count = 0;
  c->timeout_ticks = kDefaultTimeoutTicks;
  c->skew = 0;
  c->abort_dev = nullptr;
  if (w8) c->wscale_host.assign(src->weight_scales, src->weight_scales + (size_t)L * 7 + 1);

  auto fail = [&](const char* what, hipError_t e) {
    set_err(err, "%s: %s", what, hipGetErrorString(e));
    delete c;
    return KIE_ERR_HIP;
  };
  hipError_t e;
  hipStream_t stm = c->stream;
  // workspace: exchange words and error word to zero, RoPE table, stream bases, norm gains, all by
  // kernels and device-to-device copies on the context's stream (no host staging, no memset)
  if ((e = launch_fill_zero(c->ws, c->wso.end, stm)) != hipSuccess) return fail("clear workspace", e);
  if ((e = launch_rope_table((float2*)(c->ws + c->wso.rope), s.max_seq, s.hd, s.theta, stm)) != hipSuccess)
    return fail("rope table", e);
  if ((e = launch_stream_bases(s, w8, (int64_t*)(c->ws + c->wso.wbase), stm)) != hipSuccess)
    return fail("stream bases", e);
  // the prompt pass's tile table (contexts with the prompt pass's scratch)
  if (c->wso.end > c->wso.ptab &&
      (e = launch_ptab(s, w8, (const int64_t*)(c->ws + c->wso.wbase), (int32_t*)(c->ws + c->wso.ptab), stm)) !=
          hipSuccess)
    return fail("prompt tile table", e);
  uint16_t* norms = (uint16_t*)(c->ws + c->wso.norms);
  for (int l = 0; l < L; ++l) {
    if ((e = hipMemcpyAsync(norms + (size_t)l * 2 * s.d, src->attn_norm[l], (size_t)s.d * 2, hipMemcpyDeviceToDevice,
                            stm)) != hipSuccess)
      return fail("copy norms", e);
    if ((e = hipMemcpyAsync(norms + (size_t)l * 2 * s.d + s.d, src->ffn_norm[l], (size_t)s.d * 2,
                            hipMemcpyDeviceToDevice, stm)) != hipSuccess)
      return fail("copy norms", e);
  }
  if ((e = hipMemcpyAsync(norms + (size_t)L * 2 * s.d, src->final_norm, (size_t)s.d * 2, hipMemcpyDeviceToDevice,
                          stm)) != hipSuccess)
    return fail("copy norms", e);
  // 8-bit weights: the matrix scales travel as kernel arguments (the caller's array may be freed
  // when kie_create returns), ordered after the workspace clear on the same stream
  if (w8 && (e = launch_set_floats((float*)(c->ws + c->wso.wscale), c->wscale_host.data(),
                                   (int32_t)c->wscale_host.size(), stm)) != hipSuccess)
    return fail("weight scales", e);
  // weights: per-WG token streams, then the embedding table
  const int64_t* wbase_dev = (const int64_t*)(c->ws + c->wso.wbase);
  for (int l = 0; l <= L; ++l) {
    PackArgs a;
    memset(&a, 0, sizeof a);
    a.s = s;
    a.packed = c->packed;
    a.wbase = wbase_dev;
    a.layer = l;
    a.w8 = w8 ? 1 : 0;
    if (l < L) {
      a.wq = src->wq[l];
      a.wk = src->wk[l];
      a.wv = src->wv[l];
      a.wo = src->wo[l];
      if (moe) {
        a.wrouter = src->w_router[l];
        a.egate = src->moe_gate[l];
        a.eup = src->moe_up[l];
        a.edown = src->moe_down[l];
        a.expert_offset = packed_expert_offset(s);
      } else {
        a.wgate = src->w_gate[l];
        a.wup = src->w_up[l];
        a.wdown = src->w_down[l];
      }
    } else {
      a.lm_head = src->lm_head;
    }
    if ((e = launch_pack_layer(a, stm)) != hipSuccess) return fail("pack weights", e);
    if (moe && l < L && (e = launch_pack_experts(a, stm)) != hipSuccess) return fail("pack experts", e);
  }
  if ((e = hipMemcpyAsync(c->packed + pk_embed_offset(s, w8), src->embed, (size_t)s.V * s.d * 2,
                          hipMemcpyDeviceToDevice, stm)) != hipSuccess)
    return fail("copy embedding", e);
  *out = c;
  return KIE_OK;
}

kie_status kie_create(const kie_config* cfg, const kie_weights* src, void* packed, void* kv_cache, void* workspace,
                      void* hip_stream, kie_ctx** out) {
  if (!workspace) {
    if (out) *out = nullptr;
    set_err(&g_create_error, "NULL argument");
    return KIE_ERR_INVALID_ARG;
  }
  return create_impl(cfg, src, packed, kv_cache, workspace, hip_stream, out);
}

kie_status kie_create_static(const kie_config* cfg, const kie_weights* src, void* packed, void* kv_cache,
                             void* hip_stream, kie_ctx** out) {
  const kie_status st = create_impl(cfg, src, packed, kv_cache, nullptr, hip_stream, out);
  if (st == KIE_OK) {
    std::lock_guard<std::mutex> lk(g_static_mu);
    g_static_owner[(*out)->device] = *out;
  }
  return st;
}

void kie_destroy(kie_ctx* ctx) {
  if (ctx && ctx->static_ws) {
    std::lock_guard<std::mutex> lk(g_static_mu);
    if (g_static_owner[ctx->device] == ctx) g_static_owner[ctx->device] = nullptr;
  }
  delete ctx;
}

int32_t kie_position(const kie_ctx* ctx) { return ctx ? ctx->pos : -1; }

kie_status kie_reset(kie_ctx* ctx) {
  if (!ctx) return KIE_ERR_INVALID_ARG;
  if (!static_owner_ok(ctx)) {
    set_err(&ctx->last_error, "another context now uses this GPU's static workspace");
    return KIE_ERR_STATE;
  }
  HIP_TRY(&ctx->last_error, hipSetDevice(ctx->device));
  HIP_TRY(&ctx->last_error, launch_fill_zero(ctx->ws + ctx->wso.err, 4, ctx->stream));
  ctx->pos = 0;
  ctx->bad_state = false;
  ctx->last_error.clear();
  return KIE_OK;
}

kie_status kie_set_token_stream(kie_ctx* ctx, int32_t* ring_host, int32_t capacity) {
  if (!ctx) return KIE_ERR_INVALID_ARG;
  if (!ring_host) {
    ctx->tok_ring = nullptr;
    ctx->ring_cap = 0;
    ctx->ring_count = 0;
    return KIE_OK;
  }
  if (capacity <= 0) {
    set_err(&ctx->last_error, "token ring capacity must be positive");
    return KIE_ERR_INVALID_ARG;
  }
  void* dev = nullptr;
  const hipError_t e = hipHostGetDevicePointer(&dev, ring_host, 0);
  if (e != hipSuccess || !dev) {
    (void)hipGetLastError();
    set_err(&ctx->last_error, "the token ring is not pinned host memory the GPU can write");
    return KIE_ERR_INVALID_ARG;
  }
  ring_host[0] = 0;
  ctx->tok_ring = (int32_t*)dev;
  ctx->ring_cap = capacity;
  ctx->ring_count = 0;
  return KIE_OK;
}

kie_status kie_set_abort_flag(kie_ctx* ctx, int32_t* host_word) {
  if (!ctx) return KIE_ERR_INVALID_ARG;
  if (!host_word) {
    ctx->abort_dev = nullptr;
    return KIE_OK;
  }
  void* dev = nullptr;
  const hipError_t e = hipHostGetDevicePointer(&dev, host_word, 0);
  if (e != hipSuccess || !dev) {
    (void)hipGetLastError();
    set_err(&ctx->last_error, "the abort word is not pinned host memory the GPU can read");
    return KIE_ERR_INVALID_ARG;
  }
  ctx->abort_dev = (int32_t*)dev;
  return KIE_OK;
}

kie_status kie_set_position(kie_ctx* ctx, int32_t pos) {
  if (!ctx) return KIE_ERR_INVALID_ARG;
  if (pos < 0 || pos > ctx->s.max_seq) {
    set_err(&ctx->last_error, "position %d outside [0, %d]", pos, ctx->s.max_seq);
    return KIE_ERR_INVALID_ARG;
  }
  ctx->pos = pos;
  return KIE_OK;
}

kie_status kie_sync(kie_ctx* ctx) {
  if (!ctx) return KIE_ERR_INVALID_ARG;
  HIP_TRY(&ctx->last_error, hipSetDevice(ctx->device));
  HIP_TRY(&ctx->last_error, hipStreamSynchronize(ctx->stream));
  uint32_t errw = 0;
  HIP_TRY(&ctx->last_error, hipMemcpy(&errw, ctx->ws + ctx->wso.err, 4, hipMemcpyDeviceToHost));
  if (errw & KERR_ABORTED) {
    ctx->bad_state = true;
    set_err(&ctx->last_error, "the launch stopped at the host's abort word (error word 0x%x)", errw);
    return KIE_ERR_ABORTED;
  }
  if (errw & KERR_TIMEOUT) {
    ctx->bad_state = true;
    set_err(&ctx->last_error, "device wait timed out (error word 0x%x)", errw);
    return KIE_ERR_TIMEOUT;
  }
  if (errw & KERR_BAD_TOKEN) {
    ctx->bad_state = true;
    set_err(&ctx->last_error, "an input token id was out of range (replaced by 0)");
    return KIE_ERR_ABORTED;
  }
  return KIE_OK;
}

static kie_status check_sampling(kie_ctx* ctx, const kie_sampling* smp) {
  const int32_t top_k = smp && smp->top_k > 1 ? smp->top_k : 1;
  if (top_k > 1) {
    if (top_k > kMaxTopK || top_k > ctx->s.V) {
      set_err(&ctx->last_error, "top_k %d exceeds the supported maximum %d or the vocabulary", top_k, kMaxTopK);
      return KIE_ERR_UNSUPPORTED;
    }
    if (!(smp->temperature > 0.f) || !(smp->temperature < INFINITY)) {
      set_err(&ctx->last_error, "temperature must be positive and finite for top-k sampling");
      return KIE_ERR_INVALID_ARG;
    }
    if (topk_merge_floats(ctx->s, top_k) > topk_capacity_floats(ctx->s)) {
      set_err(&ctx->last_error, "top_k %d does not fit this model's on-chip merge space", top_k);
      return KIE_ERR_UNSUPPORTED;
    }
  }
  return KIE_OK;
}

static kie_status launch(kie_ctx* ctx, const int32_t* first, int32_t n, const int32_t* forced, int32_t* toks_out,
                         int32_t* last_tok, float* logits, int lm_last_only, const kie_sampling* smp) {
  if (ctx->bad_state) {
    set_err(&ctx->last_error, "context holds a device error; call kie_reset");
    return KIE_ERR_STATE;
  }
  if (!static_owner_ok(ctx)) {
    set_err(&ctx->last_error, "another context now uses this GPU's static workspace");
    return KIE_ERR_STATE;
  }
  if (!first || n <= 0) {
    set_err(&ctx->last_error, "first token pointer is NULL or n <= 0");
    return KIE_ERR_INVALID_ARG;
  }
  const kie_status sst = check_sampling(ctx, smp);
  if (sst != KIE_OK) return sst;
  const int32_t top_k = smp && smp->top_k > 1 ? smp->top_k : 1;
  if ((int64_t)ctx->pos + n > ctx->s.max_seq) {
    set_err(&ctx->last_error, "position %d + %d tokens exceeds max_seq_len %d", ctx->pos, n, ctx->s.max_seq);
    return KIE_ERR_CAPACITY;
  }
  HIP_TRY(&ctx->last_error, hipSetDevice(ctx->device));
  KParams P;
  P.s = ctx->s;
  P.exo = ctx->exo;
  P.packed = ctx->packed;
  P.embed = (const uint16_t*)(ctx->packed + pk_embed_offset(ctx->s, ctx->w8));
  P.norms = (const uint16_t*)(ctx->ws + ctx->wso.norms);
  P.kv = ctx->kv;
  P.ex = (uint64_t*)(ctx->ws + ctx->wso.exch);
  P.rope = (const float2*)(ctx->ws + ctx->wso.rope);
  P.wbase = (const int64_t*)(ctx->ws + ctx->wso.wbase);
  P.err = (uint32_t*)(ctx->ws + ctx->wso.err);
  P.trace = (uint64_t*)(ctx->ws + ctx->wso.trace);
  P.first_tok = first;
  P.forced = forced;
  P.tokens_out = toks_out;
  P.last_tok_out = last_tok;
  P.logits_out = logits;
  P.pos0 = ctx->pos;
  P.n_steps = n;
  P.epoch0 = ctx->epoch;
  P.lm_last_only = lm_last_only;
  P.tok_ring = lm_last_only ? nullptr : ctx->tok_ring;
  P.ring_cap = ctx->ring_cap;
  P.ring_base = ctx->ring_count;
  P.top_k = top_k;
  P.temperature = top_k > 1 ? smp->temperature : 1.0f;
  P.seed = smp ? smp->seed : 0;
  P.timeout_ticks = ctx->timeout_ticks;
  P.abort_word = ctx->abort_dev;
  P.skew = ctx->skew;
  P.xb_lds = (uint32_t)lds_slot_offset(ctx->s);
  P.wscale = ctx->w8 ? (const float*)(ctx->ws + ctx->wso.wscale) : nullptr;
  void* args[] = {&P};
  const void* fn = (const void*)(lm_last_only ? ctx->prompt_kernel : ctx->kernel);
  HIP_TRY(&ctx->last_error,
          hipLaunchCooperativeKernel(fn, dim3(ctx->s.nwg), dim3(kThreads), args, (unsigned)ctx->lds, ctx->stream));
  ctx->pos += n;
  if (P.tok_ring) ctx->ring_count += n;
  ctx->epoch += (uint32_t)n;
  if (ctx->epoch == 0) ctx->epoch = 1;
  return KIE_OK;
}

kie_status kie_prefill(kie_ctx* ctx, const int32_t* tokens_dev, int32_t n_tokens, int32_t* first_token_dev,
                       float* last_logits_dev, const kie_sampling* sampling) {
  if (!ctx) return KIE_ERR_INVALID_ARG;
  if (!tokens_dev || !first_token_dev || n_tokens <= 0) {
    set_err(&ctx->last_error, "prefill needs tokens, an output token and n_tokens > 0");
    return KIE_ERR_INVALID_ARG;
  }
  if (ctx->bad_state) {
    set_err(&ctx->last_error, "context holds a device error; call kie_reset");
    return KIE_ERR_STATE;
  }
  const kie_status sst = check_sampling(ctx, sampling);
  if (sst != KIE_OK) return sst;
  if ((int64_t)ctx->pos + n_tokens > ctx->s.max_seq) {
    set_err(&ctx->last_error, "position %d + %d tokens exceeds max_seq_len %d", ctx->pos, n_tokens, ctx->s.max_seq);
    return KIE_ERR_CAPACITY;
  }
  // contexts on the static workspace (which has no room for the matrix-core pass's scratch), and
  // shapes the matrix-core pass does not handle: every position through the decode program,
  // teacher-forced (position i + 1 processes tokens[i + 1]); the LM head and the sampler run on
  // the last one only
  if (ctx->static_ws || !prefill_supports(ctx->s))
    return launch(ctx, tokens_dev, n_tokens, tokens_dev + 1, nullptr, first_token_dev, last_logits_dev, 1, sampling);
  // all but the last prompt position: every layer as GEMMs on the matrix cores (K/V rows only)
  if (n_tokens > 1) {
    HIP_TRY(&ctx->last_error, hipSetDevice(ctx->device));
    PrefillArgs a;
    a.s = ctx->s;
    a.packed = ctx->packed;
    a.wbase = (const int64_t*)(ctx->ws + ctx->wso.wbase);
    a.embed = (const uint16_t*)(ctx->packed + pk_embed_offset(ctx->s, ctx->w8));
    a.norms = (const uint16_t*)(ctx->ws + ctx->wso.norms);
    a.rope = (const float2*)(ctx->ws + ctx->wso.rope);
    a.kv = ctx->kv;
    a.err = (uint32_t*)(ctx->ws + ctx->wso.err);
    a.tokens = tokens_dev;
    a.x = (float*)(ctx->ws + ctx->wso.px);
    a.a3 = (uint16_t*)(ctx->ws + ctx->wso.pa3);
    a.h2 = (uint16_t*)(ctx->ws + ctx->wso.ph2);
    a.a_part = (int64_t)kPrefillChunk * prefill_kmax(ctx->s);
    a.c = (float*)(ctx->ws + ctx->wso.pc);
    a.q = (float*)(ctx->ws + ctx->wso.pq);
    a.attn_part = (float*)(ctx->ws + ctx->wso.pattn);
    a.wscale = ctx->w8 ? (const float*)(ctx->ws + ctx->wso.wscale) : nullptr;
    a.ptab = (const int32_t*)(ctx->ws + ctx->wso.ptab);
    a.rlogits = a.wt = a.ey = nullptr;
    a.sel = a.place = a.lists = a.counts = a.offs = nullptr;
    if (ctx->s.moe()) {  // the experts' scratch
      const MoePrefill m = moe_prefill_layout(ctx->s);
      uint8_t* mb = ctx->ws + ctx->wso.pmoe;
      a.rlogits = (float*)(mb + m.logits);
      a.sel = (int32_t*)(mb + m.sel);
      a.wt = (float*)(mb + m.wt);
      a.place = (int32_t*)(mb + m.place);
      a.lists = (int32_t*)(mb + m.lists);
      a.counts = (int32_t*)(mb + m.counts);
      a.offs = (int32_t*)(mb + m.offs);
      a.ey = (float*)(mb + m.y);
    }
    HIP_TRY(&ctx->last_error, launch_prefill(a, ctx->pos, n_tokens - 1, ctx->stream));
    ctx->pos += n_tokens - 1;
  }
  // the last position through the decode program: its K/V rows, the logits and the first token
  return launch(ctx, tokens_dev + (n_tokens - 1), 1, nullptr, nullptr, first_token_dev, last_logits_dev, 1, sampling);
}

kie_status kie_decode_step(kie_ctx* ctx, const int32_t* token_in_dev, const kie_sampling* sampling,
                           int32_t* token_out_dev, float* logits_dev) {
  if (!ctx) return KIE_ERR_INVALID_ARG;
  if (!token_out_dev) {
    set_err(&ctx->last_error, "token_out_dev is NULL");
    return KIE_ERR_INVALID_ARG;
  }
  return launch(ctx, token_in_dev, 1, nullptr, token_out_dev, nullptr, logits_dev, 0, sampling);
}

kie_status kie_generate(kie_ctx* ctx, const int32_t* first_token_dev, int32_t n_steps, const kie_sampling* sampling,
                        const int32_t* forced_dev, int32_t* tokens_out_dev, float* logits_dev) {
  if (!ctx) return KIE_ERR_INVALID_ARG;
  if (!tokens_out_dev) {
    set_err(&ctx->last_error, "tokens_out_dev is NULL");
    return KIE_ERR_INVALID_ARG;
  }
  return launch(ctx, first_token_dev, n_steps, forced_dev, tokens_out_dev, nullptr, logits_dev, 0, sampling);
}

// ------------------------------------------------------------------ measurement helpers
kie_status kie_stream_copy(void* dst, const void* src, size_t bytes, void* hip_stream) {
  if (!dst || !src || bytes % 16 || !aligned16(dst) || !aligned16(src)) return KIE_ERR_INVALID_ARG;
  int n = 0;
  if (query_cus(&n, nullptr) != KIE_OK) return KIE_ERR_HIP;
  return launch_stream_copy(dst, src, (int64_t)bytes, n, (hipStream_t)hip_stream) == hipSuccess ? KIE_OK : KIE_ERR_HIP;
}

kie_status kie_stream_read(const void* src, size_t bytes, uint32_t* sink_dev, void* hip_stream) {
  if (!src || !sink_dev || bytes % 16 || !aligned16(src)) return KIE_ERR_INVALID_ARG;
  int n = 0;
  if (query_cus(&n, nullptr) != KIE_OK) return KIE_ERR_HIP;
  return launch_stream_read(src, (int64_t)bytes, sink_dev, n, (hipStream_t)hip_stream) == hipSuccess ? KIE_OK
                                                                                                       : KIE_ERR_HIP;
}

kie_status kie_set_skew(kie_ctx* ctx, uint32_t level) {
  if (!ctx) return KIE_ERR_INVALID_ARG;
  if (level > 64) {
    set_err(&ctx->last_error, "skew level %u is above 64", level);
    return KIE_ERR_INVALID_ARG;
  }
  ctx->skew = level;
  return KIE_OK;
}

kie_status kie_set_wait_timeout(kie_ctx* ctx, uint64_t microseconds) {
  if (!ctx) return KIE_ERR_INVALID_ARG;
  if (microseconds > (uint64_t)3600 * 1000000) {
    set_err(&ctx->last_error, "wait timeout above one hour");
    return KIE_ERR_INVALID_ARG;
  }
  ctx->timeout_ticks = microseconds == 0 ? kDefaultTimeoutTicks : (int64_t)microseconds * 100;
  return KIE_OK;
}

int64_t kie_trace_offset(const kie_config* cfg) {
  Shape s;
  if (make_shape(cfg, 0, &s, nullptr) != KIE_OK) return -1;
  return workspace_layout(s).trace;
}

}  // extern "C"
