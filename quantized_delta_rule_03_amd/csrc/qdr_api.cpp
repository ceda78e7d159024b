// qdr_api.cpp -- C ABI of libqdr (declared in include/qdr.h): argument validation,
// layout/metadata construction, kernel selection. No allocation, no synchronization.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qdr.h"
#include "qdr_internal.h"

namespace {

#define CHECK(expr)        \
  do {                     \
    int rc_ = (expr);      \
    if (rc_) return rc_;   \
  } while (0)

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return QDR_OK;
}

// Host view of one head's layout (the same rules as the format in include/qdr.h).
struct HeadLayout {
  uint32_t tile_bytes;
  uint8_t seg_bits[4];
  uint8_t perm[qdr::kD];
  bool identity;
};

int head_layout(const uint8_t* bits, HeadLayout* out, int h) {
  static const int widths[3] = {8, 6, 4};
  int p = 0;
  uint32_t bytes = 0;
  for (int wi = 0; wi < 3; ++wi) {
    int count = 0;
    for (int j = 0; j < qdr::kD; ++j) {
      const int b = bits[j];
      if (b != 4 && b != 6 && b != 8)
        return fail(QDR_EUNSUPPORTED, "bits[%d][%d] = %d is not 4, 6 or 8", h, j, b);
      if (b == widths[wi]) {
        out->perm[p++] = (uint8_t)j;
        ++count;
      }
    }
    if (count % qdr::kSeg)
      return fail(QDR_EUNSUPPORTED, "head %d has %d channels of width %d (not a multiple of 32)",
                  h, count, widths[wi]);
    bytes += (uint32_t)(qdr::kD * count * widths[wi] / 8);
  }
  for (int s = 0; s < 4; ++s) out->seg_bits[s] = bits[out->perm[s * qdr::kSeg]];
  out->identity = true;
  for (int q = 0; q < qdr::kD; ++q) out->identity = out->identity && out->perm[q] == q;
  out->tile_bytes = bytes;
  return QDR_OK;
}

struct Geometry {
  std::vector<HeadLayout> heads;
  std::vector<uint32_t> off;
  std::vector<uint16_t> order;  // heads by width 8, 6, 4 (uniform heads)
  uint32_t req_bytes = 0;
  bool uniform = true;
  int n_class[3] = {0, 0, 0};
};

int check_scalars(const qdr_desc* d) {
  if (!d) return fail(QDR_EINVAL, "desc is NULL");
  if (d->n_req < 0) return fail(QDR_EINVAL, "n_req = %d < 0", d->n_req);
  if (d->n_head < 1 || d->n_head > 1024)
    return fail(QDR_EINVAL, "n_head = %d outside [1, 1024]", d->n_head);
  if (d->dk != qdr::kD || d->dv != qdr::kD)
    return fail(QDR_EUNSUPPORTED, "dk = %d, dv = %d: only 128 x 128 states are supported", d->dk,
                d->dv);
  if (d->gate != QDR_GATE_GDN && d->gate != QDR_GATE_KDA)
    return fail(QDR_EINVAL, "gate = %d is neither GDN (0) nor KDA (1)", d->gate);
  if (!d->bits) return fail(QDR_EINVAL, "desc->bits is NULL");
  if (d->window < 0) return fail(QDR_EINVAL, "window = %d < 0", d->window);
  if (d->rule < QDR_RULE_STEP || d->rule > QDR_RULE_TENSOR)
    return fail(QDR_EINVAL, "rule = %d is not a QDR_RULE_* value", d->rule);
  if ((long long)d->n_req * d->n_head > (1LL << 31) - 1)
    return fail(QDR_EINVAL, "n_req * n_head overflows");
  return QDR_OK;
}

int check_desc(const qdr_desc* d, Geometry* g) {
  CHECK(check_scalars(d));
  if (g) {
    g->heads.resize(d->n_head);
    g->off.resize(d->n_head);
    uint64_t off = 0;
    for (int h = 0; h < d->n_head; ++h) {
      int rc = head_layout(d->bits + (size_t)h * qdr::kD, &g->heads[h], h);
      if (rc) return rc;
      g->off[h] = (uint32_t)off;
      off += g->heads[h].tile_bytes;
    }
    if (off > 0xFFFFFFFFull) return fail(QDR_EINVAL, "request too large");
    g->req_bytes = (uint32_t)off;
    static const int widths[3] = {8, 6, 4};
    for (int h = 0; h < d->n_head; ++h) {
      const uint8_t* sb = g->heads[h].seg_bits;
      g->uniform = g->uniform && sb[0] == sb[1] && sb[1] == sb[2] && sb[2] == sb[3];
    }
    g->order.clear();
    for (int c = 0; c < 3; ++c) {
      g->n_class[c] = 0;
      for (int h = 0; h < d->n_head; ++h)
        if (g->heads[h].seg_bits[0] == widths[c] && g->heads[h].seg_bits[3] == widths[c]) {
          g->order.push_back((uint16_t)h);
          ++g->n_class[c];
        }
    }
  }
  return QDR_OK;
}

// What the launches need from a bit map: the request stride and the width classes.
struct Summary {
  uint32_t req_bytes = 0;
  bool uniform = true;
  int n_class[3] = {0, 0, 0};
};

// Summaries of the last few validated bit maps. A call whose bit map equals a cached one
// (compared in full, so an edited map is never mistaken for a cached one) skips the
// per-head layout pass and allocates nothing; a miss validates the map, summarises it
// and replaces the oldest entry.
struct CacheEntry {
  int32_t n_head = 0;
  std::vector<uint8_t> bits;
  Summary sum;
};
constexpr int kCacheEntries = 8;
std::mutex g_cache_mu;
CacheEntry g_cache[kCacheEntries];
int g_cache_next = 0;

int check_desc_summary(const qdr_desc* d, Summary* out) {
  CHECK(check_scalars(d));
  const size_t nb = (size_t)d->n_head * qdr::kD;
  {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    for (const CacheEntry& e : g_cache)
      if (e.n_head == d->n_head && memcmp(e.bits.data(), d->bits, nb) == 0) {
        *out = e.sum;
        return QDR_OK;
      }
  }
  Geometry g;
  CHECK(check_desc(d, &g));
  Summary sm;
  sm.req_bytes = g.req_bytes;
  sm.uniform = g.uniform;
  for (int c = 0; c < 3; ++c) sm.n_class[c] = g.n_class[c];
  std::lock_guard<std::mutex> lk(g_cache_mu);
  CacheEntry& e = g_cache[g_cache_next];
  g_cache_next = (g_cache_next + 1) % kCacheEntries;
  e.n_head = d->n_head;
  e.bits.assign(d->bits, d->bits + nb);
  e.sum = sm;
  *out = sm;
  return QDR_OK;
}

int check_ptr(const void* p, const char* name, bool required) {
  if (!p) return required ? fail(QDR_EINVAL, "%s is NULL", name) : QDR_OK;
  if (reinterpret_cast<uintptr_t>(p) & 15u)
    return fail(QDR_EALIGN, "%s = %p is not 16-byte aligned", name, p);
  return QDR_OK;
}

qdr::Pool pool_of(const qdr_desc* d, const void* meta, const Summary& g) {
  qdr::Pool p;
  p.meta = meta;
  p.n_head = d->n_head;
  p.n_unit = d->n_req * d->n_head;
  p.req_bytes = g.req_bytes;
  p.uniform = g.uniform ? 1 : 0;
  for (int c = 0; c < 3; ++c) p.n_class[c] = g.n_class[c];
  p.rule = d->rule;
  return p;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QDR_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

struct RankItem {
  double tau;
  int idx;
};

void quartile(int n, const double* tau, uint8_t* out) {
  std::vector<RankItem> it(n);
  for (int i = 0; i < n; ++i) it[i] = {tau[i], i};
  std::stable_sort(it.begin(), it.end(),
                   [](const RankItem& a, const RankItem& b) { return a.tau < b.tau; });
  const int quarter = n / 4;
  for (int r = 0; r < n; ++r)
    out[it[r].idx] = (uint8_t)(r < quarter ? 4 : (r >= n - quarter ? 8 : 6));
}

}  // namespace

// ---- window mode without a caller workspace ---------------------------------------
// The window buffer of qdr_decode_window_static: a fixed device array of the library
// (one per GPU, held until the process ends), for callers that cannot allocate. Its
// device address comes from hipGetSymbolAddress, once per device, and only that address
// is handed to the kernels (the array's name is a host-side stand-in in host code).
constexpr size_t kStaticWindowBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticWindowBytes];
constexpr int kScratchDevices = 64;
static void* g_scratch_ptr[kScratchDevices];
static std::mutex g_scratch_mu;

static int static_window_buffer(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "qdr_decode_window_static: hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(QDR_EUNSUPPORTED, "qdr_decode_window_static: device %d beyond %d", dev,
                kScratchDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                        "qdr_decode_window_static: hipGetSymbolAddress");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QDR_OK;
}

extern "C" {

int qdr_assign_bits(int32_t gate, int32_t n_head, int32_t dk, const double* halflife,
                    uint8_t* bits_out) {
  if (n_head < 1 || dk < 1 || !halflife || !bits_out)
    return fail(QDR_EINVAL, "qdr_assign_bits: bad arguments");
  if (gate == QDR_GATE_GDN) {
    std::vector<uint8_t> hb(n_head);
    quartile(n_head, halflife, hb.data());
    for (int h = 0; h < n_head; ++h) memset(bits_out + (size_t)h * dk, hb[h], (size_t)dk);
    return ok();
  }
  if (gate == QDR_GATE_KDA) {
    for (int h = 0; h < n_head; ++h)
      quartile(dk, halflife + (size_t)h * dk, bits_out + (size_t)h * dk);
    return ok();
  }
  return fail(QDR_EINVAL, "qdr_assign_bits: gate = %d", gate);
}

int qdr_state_bytes(const qdr_desc* d, size_t* packed, size_t* scales, size_t* meta,
                    size_t* window_buf) {
  Summary g;
  CHECK(check_desc_summary(d, &g));
  const size_t n_unit = (size_t)d->n_req * d->n_head;
  if (packed) *packed = (size_t)d->n_req * g.req_bytes;
  if (scales) *scales = n_unit * qdr::kD * sizeof(float);
  if (meta) *meta = qdr::meta_bytes(d->n_head);
  if (window_buf) *window_buf = d->window > 0 ? n_unit * qdr::window_unit_bytes(d->window) : 0;
  return ok();
}

int qdr_init_state(const qdr_desc* d, void* packed, float* row_scale, float* col_scale,
                   void* meta, void* stream) {
  Geometry g;
  CHECK(check_desc(d, &g));
  const bool any = d->n_req > 0;
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(packed, "packed", any));
  CHECK(check_ptr(row_scale, "row_scale", any));
  CHECK(check_ptr(col_scale, "col_scale", any));
  std::vector<uint8_t> host(qdr::meta_bytes(d->n_head), 0);
  auto* hdr = reinterpret_cast<qdr::MetaHeader*>(host.data());
  hdr->magic = qdr::kMetaMagic;
  hdr->n_head = (uint32_t)d->n_head;
  hdr->dk = (uint32_t)d->dk;
  hdr->dv = (uint32_t)d->dv;
  hdr->gate = (uint32_t)d->gate;
  hdr->req_bytes = g.req_bytes;
  hdr->window = (uint32_t)d->window;
  hdr->uniform = g.uniform ? 1u : 0u;
  for (int c = 0; c < 3; ++c) hdr->n_class[c] = (uint32_t)g.n_class[c];
  auto* mh = reinterpret_cast<qdr::MetaHead*>(host.data() + sizeof(qdr::MetaHeader));
  for (int h = 0; h < d->n_head; ++h) {
    mh[h].tile_off = g.off[h];
    mh[h].tile_bytes = g.heads[h].tile_bytes;
    memcpy(mh[h].seg_bits, g.heads[h].seg_bits, 4);
    mh[h].identity = g.heads[h].identity ? 1u : 0u;
    memcpy(mh[h].perm, g.heads[h].perm, qdr::kD);
    for (int q = 0; q < qdr::kD; ++q) mh[h].iperm[g.heads[h].perm[q]] = (uint8_t)q;
  }
  if (g.uniform) {
    uint16_t* ord = reinterpret_cast<uint16_t*>(host.data() + sizeof(qdr::MetaHeader) +
                                                (size_t)d->n_head * sizeof(qdr::MetaHead));
    for (size_t i = 0; i < g.order.size(); ++i) ord[i] = g.order[i];
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the table is small; a synchronous copy keeps the host vector's lifetime simple
  hipError_t e = hipMemcpyAsync(meta, host.data(), host.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "qdr_init_state: metadata copy");
  Summary sm;
  sm.req_bytes = g.req_bytes;
  sm.uniform = g.uniform;
  for (int c = 0; c < 3; ++c) sm.n_class[c] = g.n_class[c];
  return hip_status(qdr::launch_init(pool_of(d, meta, sm), static_cast<uint8_t*>(packed),
                                     row_scale, col_scale, s),
                    "qdr_init_state: launch");
}

int qdr_quantize_state(const qdr_desc* d, const void* meta, const float* S, void* packed,
                       float* row_scale, float* col_scale, void* stream) {
  Summary g;
  CHECK(check_desc_summary(d, &g));
  const bool any = d->n_req > 0;
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(S, "S", any));
  CHECK(check_ptr(packed, "packed", any));
  CHECK(check_ptr(row_scale, "row_scale", any));
  CHECK(check_ptr(col_scale, "col_scale", any));
  return hip_status(qdr::launch_quantize(pool_of(d, meta, g), S, static_cast<uint8_t*>(packed),
                                         row_scale, col_scale, static_cast<hipStream_t>(stream)),
                    "qdr_quantize_state: launch");
}

int qdr_dequantize_state(const qdr_desc* d, const void* meta, const void* packed,
                         const float* row_scale, const float* col_scale, float* S_out,
                         void* stream) {
  Summary g;
  CHECK(check_desc_summary(d, &g));
  const bool any = d->n_req > 0;
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(packed, "packed", any));
  CHECK(check_ptr(row_scale, "row_scale", any));
  CHECK(check_ptr(col_scale, "col_scale", any));
  CHECK(check_ptr(S_out, "S_out", any));
  return hip_status(qdr::launch_dequantize(pool_of(d, meta, g),
                                           static_cast<const uint8_t*>(packed), row_scale,
                                           col_scale, S_out, static_cast<hipStream_t>(stream)),
                    "qdr_dequantize_state: launch");
}

int qdr_decode_step(const qdr_desc* d, const void* meta, void* packed, float* row_scale,
                    float* col_scale, const float* q, const float* k, const float* v,
                    const float* a, const float* b, float* o, void* stream) {
  Summary g;
  CHECK(check_desc_summary(d, &g));
  const bool any = d->n_req > 0;
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(packed, "packed", any));
  CHECK(check_ptr(row_scale, "row_scale", any));
  CHECK(check_ptr(col_scale, "col_scale", any));
  CHECK(check_ptr(q, "q", any));
  CHECK(check_ptr(k, "k", any));
  CHECK(check_ptr(v, "v", any));
  CHECK(check_ptr(a, "a", any));
  CHECK(check_ptr(b, "b", any));
  CHECK(check_ptr(o, "o", any));
  return hip_status(qdr::launch_step(pool_of(d, meta, g), d->gate, static_cast<uint8_t*>(packed),
                                     row_scale, col_scale, q, k, v, a, b, o,
                                     static_cast<hipStream_t>(stream)),
                    "qdr_decode_step: launch");
}

int qdr_decode_window(const qdr_desc* d, const void* meta, void* packed, float* row_scale,
                      float* col_scale, void* window_buf, int32_t t, const float* q,
                      const float* k, const float* v, const float* a, const float* b,
                      float* o, void* stream) {
  Summary g;
  CHECK(check_desc_summary(d, &g));
  if (d->window < 1) return fail(QDR_EUNSUPPORTED, "desc->window = %d: no window mode", d->window);
  if (d->rule != QDR_RULE_STEP)
    return fail(QDR_EUNSUPPORTED, "window mode takes only QDR_RULE_STEP (rule = %d)", d->rule);
  if (d->window > qdr::kWindowMax)
    return fail(QDR_EUNSUPPORTED, "desc->window = %d exceeds %d", d->window, qdr::kWindowMax);
  if (t < 0 || t >= d->window)
    return fail(QDR_EUNSUPPORTED, "window position t = %d outside [0, %d)", t, d->window);
  const bool any = d->n_req > 0;
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(packed, "packed", any));
  CHECK(check_ptr(row_scale, "row_scale", any));
  CHECK(check_ptr(col_scale, "col_scale", any));
  CHECK(check_ptr(window_buf, "window_buf", any));
  CHECK(check_ptr(q, "q", any));
  CHECK(check_ptr(k, "k", any));
  CHECK(check_ptr(v, "v", any));
  CHECK(check_ptr(a, "a", any));
  CHECK(check_ptr(b, "b", any));
  CHECK(check_ptr(o, "o", any));
  return hip_status(qdr::launch_window(pool_of(d, meta, g), d->gate, d->window, t,
                                       static_cast<uint8_t*>(packed), row_scale, col_scale,
                                       static_cast<uint8_t*>(window_buf), q, k, v, a, b, o, 0,
                                       nullptr, nullptr, static_cast<hipStream_t>(stream)),
                    "qdr_decode_window: launch");
}

int qdr_decode_window_static(const qdr_desc* d, const void* meta, void* packed,
                             float* row_scale, float* col_scale, int32_t t, const float* q,
                             const float* k, const float* v, const float* a, const float* b,
                             float* o, void* stream) {
  Summary g;
  CHECK(check_desc_summary(d, &g));
  if (d->window < 1) return fail(QDR_EUNSUPPORTED, "desc->window = %d: no window mode", d->window);
  if (d->rule != QDR_RULE_STEP)
    return fail(QDR_EUNSUPPORTED, "window mode takes only QDR_RULE_STEP (rule = %d)", d->rule);
  if (d->window > qdr::kWindowMax)
    return fail(QDR_EUNSUPPORTED, "desc->window = %d exceeds %d", d->window, qdr::kWindowMax);
  if (t < 0 || t >= d->window)
    return fail(QDR_EUNSUPPORTED, "window position t = %d outside [0, %d)", t, d->window);
  const size_t need = (size_t)d->n_req * d->n_head * qdr::window_unit_bytes(d->window);
  if (need > kStaticWindowBytes)
    return fail(QDR_EUNSUPPORTED,
                "qdr_decode_window_static: the window buffer needs %zu bytes, more than the "
                "library's static %zu bytes (use qdr_decode_window with a caller buffer)",
                need, kStaticWindowBytes);
  const bool any = d->n_req > 0;
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(packed, "packed", any));
  CHECK(check_ptr(row_scale, "row_scale", any));
  CHECK(check_ptr(col_scale, "col_scale", any));
  CHECK(check_ptr(q, "q", any));
  CHECK(check_ptr(k, "k", any));
  CHECK(check_ptr(v, "v", any));
  CHECK(check_ptr(a, "a", any));
  CHECK(check_ptr(b, "b", any));
  CHECK(check_ptr(o, "o", any));
  if (!any) return ok();
  void* buf = nullptr;
  CHECK(static_window_buffer(&buf));
  return hip_status(qdr::launch_window(pool_of(d, meta, g), d->gate, d->window, t,
                                       static_cast<uint8_t*>(packed), row_scale, col_scale,
                                       static_cast<uint8_t*>(buf), q, k, v, a, b, o, 0, nullptr,
                                       nullptr, static_cast<hipStream_t>(stream)),
                    "qdr_decode_window_static: launch");
}

int qdr_decode_chunk(const qdr_desc* d, const void* meta, void* packed, float* row_scale,
                     float* col_scale, int32_t T, const float* q, const float* k, const float* v,
                     const float* a, const float* b, float* o, void* stream) {
  Summary g;
  CHECK(check_desc_summary(d, &g));
  if (T < 0) return fail(QDR_EINVAL, "T = %d is negative", T);
  if (d->rule != QDR_RULE_STEP)
    return fail(QDR_EUNSUPPORTED, "chunk mode takes only QDR_RULE_STEP (rule = %d)", d->rule);
  const bool any = d->n_req > 0 && T > 0;
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(packed, "packed", any));
  CHECK(check_ptr(row_scale, "row_scale", any));
  CHECK(check_ptr(col_scale, "col_scale", any));
  CHECK(check_ptr(q, "q", any));
  CHECK(check_ptr(k, "k", any));
  CHECK(check_ptr(v, "v", any));
  CHECK(check_ptr(a, "a", any));
  CHECK(check_ptr(b, "b", any));
  CHECK(check_ptr(o, "o", any));
  return hip_status(qdr::launch_chunk(pool_of(d, meta, g), d->gate, T,
                                      static_cast<uint8_t*>(packed), row_scale, col_scale, q, k,
                                      v, a, b, o, 0, nullptr, nullptr, nullptr,
                                      static_cast<hipStream_t>(stream)),
                    "qdr_decode_chunk: launch");
}

// ---- compensator tokens ---------------------------------------------------------

static int check_comp(const qdr_desc* d, int32_t m, bool any, const void* tok_idx,
                      const void* tok_val) {
  if (m < 0 || m > qdr::kCompMax)
    return fail(QDR_EINVAL, "m = %d outside [0, %d]", m, qdr::kCompMax);
  if (d->rule != QDR_RULE_STEP)
    return fail(QDR_EUNSUPPORTED, "compensator tokens take only QDR_RULE_STEP (rule = %d)",
                d->rule);
  CHECK(check_ptr(tok_idx, "tok_idx", any && m > 0));
  CHECK(check_ptr(tok_val, "tok_val", any && m > 0));
  return QDR_OK;
}

int qdr_comp_quantize(const qdr_desc* d, const void* meta, void* packed, float* row_scale,
                      float* col_scale, int32_t m, uint16_t* tok_idx, float* tok_val,
                      const float* S_in, void* stream) {
  Summary g;
  CHECK(check_desc_summary(d, &g));
  const bool any = d->n_req > 0;
  CHECK(check_comp(d, m, any, tok_idx, tok_val));
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(packed, "packed", any));
  CHECK(check_ptr(row_scale, "row_scale", any));
  CHECK(check_ptr(col_scale, "col_scale", any));
  CHECK(check_ptr(S_in, "S_in", any));
  if (!any) return ok();
  return hip_status(qdr::launch_chunk(pool_of(d, meta, g), d->gate, 0,
                                      static_cast<uint8_t*>(packed), row_scale, col_scale,
                                      nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, m,
                                      tok_idx, tok_val, S_in, static_cast<hipStream_t>(stream)),
                    "qdr_comp_quantize: launch");
}

int qdr_comp_chunk(const qdr_desc* d, const void* meta, void* packed, float* row_scale,
                   float* col_scale, int32_t m, uint16_t* tok_idx, float* tok_val, int32_t T,
                   const float* q, const float* k, const float* v, const float* a,
                   const float* b, float* o, void* stream) {
  Summary g;
  CHECK(check_desc_summary(d, &g));
  if (T < 0) return fail(QDR_EINVAL, "T = %d is negative", T);
  const bool any = d->n_req > 0 && T > 0;
  CHECK(check_comp(d, m, any, tok_idx, tok_val));
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(packed, "packed", any));
  CHECK(check_ptr(row_scale, "row_scale", any));
  CHECK(check_ptr(col_scale, "col_scale", any));
  CHECK(check_ptr(q, "q", any));
  CHECK(check_ptr(k, "k", any));
  CHECK(check_ptr(v, "v", any));
  CHECK(check_ptr(a, "a", any));
  CHECK(check_ptr(b, "b", any));
  CHECK(check_ptr(o, "o", any));
  return hip_status(qdr::launch_chunk(pool_of(d, meta, g), d->gate, T,
                                      static_cast<uint8_t*>(packed), row_scale, col_scale, q, k,
                                      v, a, b, o, m, tok_idx, tok_val, nullptr,
                                      static_cast<hipStream_t>(stream)),
                    "qdr_comp_chunk: launch");
}

int qdr_comp_window(const qdr_desc* d, const void* meta, void* packed, float* row_scale,
                    float* col_scale, int32_t m, uint16_t* tok_idx, float* tok_val,
                    void* window_buf, int32_t t, const float* q, const float* k, const float* v,
                    const float* a, const float* b, float* o, void* stream) {
  Summary g;
  CHECK(check_desc_summary(d, &g));
  if (d->window < 1) return fail(QDR_EUNSUPPORTED, "desc->window = %d: no window mode", d->window);
  if (d->window > qdr::kWindowMax)
    return fail(QDR_EUNSUPPORTED, "desc->window = %d exceeds %d", d->window, qdr::kWindowMax);
  if (t < 0 || t >= d->window)
    return fail(QDR_EUNSUPPORTED, "window position t = %d outside [0, %d)", t, d->window);
  const bool any = d->n_req > 0;
  CHECK(check_comp(d, m, any, tok_idx, tok_val));
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(packed, "packed", any));
  CHECK(check_ptr(row_scale, "row_scale", any));
  CHECK(check_ptr(col_scale, "col_scale", any));
  CHECK(check_ptr(window_buf, "window_buf", any));
  CHECK(check_ptr(q, "q", any));
  CHECK(check_ptr(k, "k", any));
  CHECK(check_ptr(v, "v", any));
  CHECK(check_ptr(a, "a", any));
  CHECK(check_ptr(b, "b", any));
  CHECK(check_ptr(o, "o", any));
  return hip_status(qdr::launch_window(pool_of(d, meta, g), d->gate, d->window, t,
                                       static_cast<uint8_t*>(packed), row_scale, col_scale,
                                       static_cast<uint8_t*>(window_buf), q, k, v, a, b, o, m,
                                       tok_idx, tok_val, static_cast<hipStream_t>(stream)),
                    "qdr_comp_window: launch");
}

int qdr_comp_dequantize(const qdr_desc* d, const void* meta, const void* packed,
                        const float* row_scale, const float* col_scale, int32_t m,
                        const uint16_t* tok_idx, const float* tok_val, float* S_out,
                        void* stream) {
  Summary g;
  CHECK(check_desc_summary(d, &g));
  const bool any = d->n_req > 0;
  CHECK(check_comp(d, m, any, tok_idx, tok_val));
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(packed, "packed", any));
  CHECK(check_ptr(row_scale, "row_scale", any));
  CHECK(check_ptr(col_scale, "col_scale", any));
  CHECK(check_ptr(S_out, "S_out", any));
  const qdr::Pool p = pool_of(d, meta, g);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  CHECK(hip_status(qdr::launch_dequantize(p, static_cast<const uint8_t*>(packed), row_scale,
                                          col_scale, S_out, s),
                   "qdr_comp_dequantize: launch"));
  return hip_status(qdr::launch_comp_add(p.n_unit, m, tok_idx, tok_val, S_out, s),
                    "qdr_comp_dequantize: launch");
}

// ---- DAMP-style storage variant ----------------------------------------------

static int check_damp(const qdr_damp_desc* d, std::vector<uint8_t>* perm) {
  if (!d) return fail(QDR_EINVAL, "desc is NULL");
  if (d->n_req < 0) return fail(QDR_EINVAL, "n_req = %d < 0", d->n_req);
  if (d->n_head < 1 || d->n_head > 1024)
    return fail(QDR_EINVAL, "n_head = %d outside [1, 1024]", d->n_head);
  if (d->gate != QDR_GATE_GDN && d->gate != QDR_GATE_KDA)
    return fail(QDR_EINVAL, "gate = %d is neither GDN (0) nor KDA (1)", d->gate);
  if ((long long)d->n_req * d->n_head > (1LL << 31) - 1)
    return fail(QDR_EINVAL, "n_req * n_head overflows");
  if (!d->sel) return fail(QDR_EINVAL, "desc->sel is NULL");
  if (perm) perm->assign((size_t)d->n_head * qdr::kD, 0);
  for (int h = 0; h < d->n_head; ++h) {
    const uint8_t* sh = d->sel + (size_t)h * qdr::kD;
    int n = 0;
    for (int j = 0; j < qdr::kD; ++j) n += sh[j] ? 1 : 0;
    if (n != qdr::kDampHalf)
      return fail(QDR_EUNSUPPORTED, "head %d selects %d binary16 channels, not %d", h, n,
                  qdr::kDampHalf);
    if (perm) {
      uint8_t* ph = perm->data() + (size_t)h * qdr::kD;
      int a = 0, b = qdr::kDampHalf;
      for (int j = 0; j < qdr::kD; ++j) ph[sh[j] ? a++ : b++] = (uint8_t)j;
    }
  }
  return QDR_OK;
}

static qdr::DampPool damp_pool(const qdr_damp_desc* d, const void* meta) {
  int ident = 1;
  for (int h = 0; h < d->n_head && ident; ++h)
    for (int j = 0; j < qdr::kD; ++j)
      if ((d->sel[(size_t)h * qdr::kD + j] != 0) != (j < qdr::kDampHalf)) {
        ident = 0;
        break;
      }
  return {static_cast<const uint8_t*>(meta), d->n_head, d->n_req * d->n_head, d->gate, ident};
}

int qdr_damp_select(int32_t gate, int32_t n_head, const double* halflife, uint8_t* sel_out) {
  if (gate != QDR_GATE_GDN && gate != QDR_GATE_KDA)
    return fail(QDR_EINVAL, "gate = %d is neither GDN (0) nor KDA (1)", gate);
  if (n_head < 1 || n_head > 1024) return fail(QDR_EINVAL, "n_head = %d outside [1, 1024]", n_head);
  if (!halflife || !sel_out) return fail(QDR_EINVAL, "halflife or sel_out is NULL");
  for (int h = 0; h < n_head; ++h) {
    uint8_t* sh = sel_out + (size_t)h * qdr::kD;
    memset(sh, 0, qdr::kD);
    if (gate == QDR_GATE_GDN) {
      for (int j = 0; j < qdr::kDampHalf; ++j) sh[j] = 1;  // one lifetime per head
      continue;
    }
    const double* th = halflife + (size_t)h * qdr::kD;
    std::vector<int> idx(qdr::kD);
    for (int j = 0; j < qdr::kD; ++j) idx[j] = j;
    // longest-lived first, ties by channel index
    std::stable_sort(idx.begin(), idx.end(), [&](int x, int y) { return th[x] > th[y]; });
    for (int j = 0; j < qdr::kDampHalf; ++j) sh[idx[j]] = 1;
  }
  return ok();
}

int qdr_damp_bytes(const qdr_damp_desc* d, size_t* half, size_t* codes, size_t* scales,
                   size_t* meta) {
  CHECK(check_damp(d, nullptr));
  const size_t n_unit = (size_t)d->n_req * d->n_head;
  if (half) *half = n_unit * qdr::kD * qdr::kDampHalf * 2;
  if (codes) *codes = n_unit * qdr::kD * (qdr::kD - qdr::kDampHalf);
  if (scales) *scales = n_unit * (qdr::kD - qdr::kDampHalf) * sizeof(float);
  if (meta) *meta = (size_t)d->n_head * qdr::kD;
  return ok();
}

int qdr_damp_init(const qdr_damp_desc* d, void* meta, void* half, void* codes, float* R,
                  void* stream) {
  std::vector<uint8_t> perm;
  CHECK(check_damp(d, &perm));
  const bool any = d->n_req > 0;
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(half, "half", any));
  CHECK(check_ptr(codes, "codes", any));
  CHECK(check_ptr(R, "R", any));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(meta, perm.data(), perm.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "qdr_damp_init: metadata copy");
  return hip_status(qdr::launch_damp(qdr::kDampInit, damp_pool(d, meta),
                                     static_cast<uint16_t*>(half), static_cast<int8_t*>(codes),
                                     R, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, 0, 0, s),
                    "qdr_damp_init: launch");
}

int qdr_damp_quantize(const qdr_damp_desc* d, const void* meta, const float* S, void* half,
                      void* codes, float* R, uint64_t seed, uint64_t step, void* stream) {
  CHECK(check_damp(d, nullptr));
  const bool any = d->n_req > 0;
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(S, "S", any));
  CHECK(check_ptr(half, "half", any));
  CHECK(check_ptr(codes, "codes", any));
  CHECK(check_ptr(R, "R", any));
  return hip_status(qdr::launch_damp(qdr::kDampQuantize, damp_pool(d, meta),
                                     static_cast<uint16_t*>(half), static_cast<int8_t*>(codes),
                                     R, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, S,
                                     nullptr, seed, step, static_cast<hipStream_t>(stream)),
                    "qdr_damp_quantize: launch");
}

int qdr_damp_step(const qdr_damp_desc* d, const void* meta, void* half, void* codes, float* R,
                  const float* q, const float* k, const float* v, const float* a,
                  const float* b, float* o, uint64_t seed, uint64_t step, void* stream) {
  CHECK(check_damp(d, nullptr));
  const bool any = d->n_req > 0;
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(half, "half", any));
  CHECK(check_ptr(codes, "codes", any));
  CHECK(check_ptr(R, "R", any));
  CHECK(check_ptr(q, "q", any));
  CHECK(check_ptr(k, "k", any));
  CHECK(check_ptr(v, "v", any));
  CHECK(check_ptr(a, "a", any));
  CHECK(check_ptr(b, "b", any));
  CHECK(check_ptr(o, "o", any));
  return hip_status(qdr::launch_damp(qdr::kDampStep, damp_pool(d, meta),
                                     static_cast<uint16_t*>(half), static_cast<int8_t*>(codes),
                                     R, q, k, v, a, b, o, nullptr, nullptr, seed, step,
                                     static_cast<hipStream_t>(stream)),
                    "qdr_damp_step: launch");
}

int qdr_damp_dequantize(const qdr_damp_desc* d, const void* meta, const void* half,
                        const void* codes, const float* R, float* S, void* stream) {
  CHECK(check_damp(d, nullptr));
  const bool any = d->n_req > 0;
  CHECK(check_ptr(meta, "meta", true));
  CHECK(check_ptr(half, "half", any));
  CHECK(check_ptr(codes, "codes", any));
  CHECK(check_ptr(R, "R", any));
  CHECK(check_ptr(S, "S", any));
  return hip_status(qdr::launch_damp(qdr::kDampDequantize, damp_pool(d, meta),
                                     const_cast<uint16_t*>(static_cast<const uint16_t*>(half)),
                                     const_cast<int8_t*>(static_cast<const int8_t*>(codes)),
                                     const_cast<float*>(R), nullptr, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, nullptr, S, 0, 0,
                                     static_cast<hipStream_t>(stream)),
                    "qdr_damp_dequantize: launch");
}

const char* qdr_last_error(void) { return g_err.c_str(); }

}  // extern "C"
