// C ABI of libtokenswift.so: host-side validation, tree masks, launches.
// Every check happens before anything is enqueued; see include/tokenswift.h.
#include "tokenswift.h"
#include "ts_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return TS_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Ancestor-or-self masks of a token tree (TokenSwift summary, Appendix E:
// each tree token attends only to its predecessors), two 64-bit words per
// node (anc[2i] nodes 0-63, anc[2i+1] nodes 64-127). Returns false when
// parent[] is not a tree listed parents-first.
bool build_masks(const int32_t* parent, int32_t T, uint64_t* anc, char* why, size_t why_len) {
  for (int i = 0; i < 2 * TS_MAX_TREE; ++i) anc[i] = 0;
  if (parent[0] != -1) {
    snprintf(why, why_len, "parent[0] must be -1 (node 0 is the root), got %d", parent[0]);
    return false;
  }
  anc[0] = 1ull;
  for (int i = 1; i < T; ++i) {
    const int pi = parent[i];
    if (pi < 0 || pi >= i) {
      snprintf(why, why_len, "parent[%d] = %d must lie in [0, %d)", i, pi, i);
      return false;
    }
    anc[2 * i] = anc[2 * pi];
    anc[2 * i + 1] = anc[2 * pi + 1];
    anc[2 * i + (i >> 6)] |= 1ull << (i & 63);
  }
  return true;
}

// Candidate range and partial-cache row count of a selection (TokenSwift
// summary §3.3: the initial pairs are always kept, the budget's worth of
// candidates is selected, and the most recent rows are kept).
struct PartialRows {
  int32_t cand_lo, cand_hi, b_eff, n_part;
};
PartialRows partial_rows(int32_t n_ctx, int32_t n_sink, int32_t budget, int32_t n_recent) {
  PartialRows r;
  r.cand_lo = n_sink;
  r.cand_hi = (n_ctx - n_recent > n_sink) ? n_ctx - n_recent : n_sink;
  const int32_t n_cand = r.cand_hi - r.cand_lo;
  r.b_eff = budget < n_cand ? budget : n_cand;
  const int32_t n_sink_eff = n_sink < n_ctx ? n_sink : n_ctx;
  const int32_t n_rec_eff = n_ctx > r.cand_hi ? n_ctx - r.cand_hi : 0;
  r.n_part = n_sink_eff + r.b_eff + n_rec_eff;
  return r;
}

// Checks shared by the attention entry points.
int check_attention(const char* who, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const float* out, int64_t s_head, int64_t s_pos, int32_t n_ctx, int32_t T,
                    int32_t Hq, int32_t Hkv, int32_t d, float scale, int32_t n_split) {
  if (!q || !k || !v || !out) return fail(TS_EINVAL, "%s: null tensor pointer", who);
  if (d != 64 && d != 128) return fail(TS_ENOTSUP, "%s: head dim %d not supported (64 or 128)", who, d);
  if (T < 1) return fail(TS_EINVAL, "%s: need at least one query token (got %d)", who, T);
  if (T > TS_MAX_TREE) return fail(TS_ENOTSUP, "%s: %d tokens exceed the %d-node limit", who, T, TS_MAX_TREE);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return fail(TS_EINVAL, "%s: Hq=%d must be a positive multiple of Hkv=%d", who, Hq, Hkv);
  if (Hkv > 65535) return fail(TS_ENOTSUP, "%s: Hkv=%d too large", who, Hkv);
  if (n_ctx < 0) return fail(TS_EINVAL, "%s: n_ctx=%d is negative", who, n_ctx);
  if ((int64_t)n_ctx + T > (int64_t)INT32_MAX) return fail(TS_EINVAL, "%s: cache rows overflow int32", who);
  if (s_pos < d || s_pos % 8 != 0 || s_pos > (1 << 23))
    return fail(TS_EINVAL, "%s: s_pos=%lld must be >= d, a multiple of 8 and at most 2^23", who, (long long)s_pos);
  if (s_head < 0 || s_head % 8 != 0) return fail(TS_EINVAL, "%s: s_head=%lld must be >= 0 and a multiple of 8", who, (long long)s_head);
  if (Hkv > 1 && s_head == 0) return fail(TS_EINVAL, "%s: s_head=0 with %d KV heads", who, Hkv);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(TS_EINVAL, "%s: q, k, v and out must be 16-byte aligned", who);
  if (std::isnan(scale) || std::isinf(scale)) return fail(TS_EINVAL, "%s: scale is not finite", who);
  if (n_split < 0) return fail(TS_EINVAL, "%s: n_split=%d is negative", who, n_split);
  return TS_OK;
}

int run_attention(const char* who, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  int64_t s_head, int64_t s_pos, int32_t n_ctx, int32_t T, const uint64_t* anc,
                  int32_t Hq, int32_t Hkv, int32_t d, float scale, float* out, float* scores,
                  int32_t n_split, void* ws, size_t ws_bytes, void* stream) {
  const int32_t rows_total = n_ctx + T;
  const size_t need = ts::attn_workspace_bytes(rows_total, T, Hq, Hkv, d, n_split);
  if (ws_bytes < need) return fail(TS_EWORKSPACE, "%s: workspace of %zu bytes, need %zu", who, ws_bytes, need);
  if (need > 0 && (!ws || !aligned(ws, 256))) return fail(TS_EINVAL, "%s: workspace must be non-null and 256-byte aligned", who);

  ts::AttnParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.scores = scores;
  p.s_head = s_head;
  p.s_pos = s_pos;
  p.n_ctx = n_ctx;
  p.T = T;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.d = d;
  p.M = (Hq / Hkv) * T;
  ts::attn_split_plan(rows_total, T, Hq, Hkv, d, n_split, &p.n_split, &p.rows_per_split);
  if (p.n_split > 1) {
    const size_t acc_bytes = (size_t)p.n_split * Hkv * p.M * d * sizeof(uint16_t);
    p.part_acc = static_cast<uint16_t*>(ws);
    p.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + acc_bytes);
  }
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)d);
  p.scale_log2e = sc * 1.4426950408889634f;
  for (int i = 0; i < 2 * TS_MAX_TREE; ++i) p.anc[i] = anc[i];
  const hipError_t e = ts::launch_attention(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TS_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

// ---- allocation-free verification (ts_verify_attn_noalloc) ----
// The split partials live in this file-scope device array instead of a
// caller workspace: each device holds its own copy from module load until the
// process ends. Host code uses the address hipGetSymbolAddress returns for the
// current device, never the array's name (a host-side stand-in).
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The current device's copy of the scratch array (looked up once per device).
int scratch_for_current_device(const char* who, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TS_EHIP, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(TS_ENOTSUP, "%s: device %d beyond the %d supported", who, dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(TS_EHIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", who, dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TS_OK;
}

}  // namespace

extern "C" {

int ts_abi_version(void) { return 107; }

size_t ts_verify_attn_noalloc_max_scratch(void) { return NOALLOC_SCRATCH_BYTES; }

int ts_verify_attn_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t s_head, int64_t s_pos,
                           int32_t n_ctx, int32_t T, const int32_t* parent, int32_t Hq, int32_t Hkv, int32_t d,
                           float scale, float* out, int32_t n_split, void* stream) {
  const char* who = "ts_verify_attn_noalloc";
  int rc = check_attention(who, q, k, v, out, s_head, s_pos, n_ctx, T, Hq, Hkv, d, scale, n_split);
  if (rc) return rc;
  if (!parent) return fail(TS_EINVAL, "%s: parent is null", who);
  const size_t need = ts::attn_workspace_bytes(n_ctx + T, T, Hq, Hkv, d, n_split);
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(TS_EWORKSPACE, "%s: this call needs %zu bytes of scratch, beyond the library's %zu", who, need,
                NOALLOC_SCRATCH_BYTES);
  uint64_t anc[2 * TS_MAX_TREE];
  char why[160];
  if (!build_masks(parent, T, anc, why, sizeof(why))) return fail(TS_EINVAL, "%s: %s", who, why);
  void* ws = nullptr;
  if (need > 0) {
    rc = scratch_for_current_device(who, &ws);
    if (rc) return rc;
  }
  return run_attention(who, q, k, v, s_head, s_pos, n_ctx, T, anc, Hq, Hkv, d, scale, out, nullptr, n_split, ws,
                       need, stream);
}

const char* ts_last_error(void) { return g_err; }

size_t ts_verify_attn_workspace_size(int32_t n_ctx, int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                                     int32_t n_split) {
  if (n_ctx < 0 || T < 1 || T > TS_MAX_TREE || Hq < 1 || Hkv < 1 || Hq % Hkv || (d != 64 && d != 128) || n_split < 0)
    return 0;
  return ts::attn_workspace_bytes(n_ctx + T, T, Hq, Hkv, d, n_split);
}

size_t ts_draft_attn_workspace_size(int32_t n_part, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t d,
                                    int32_t n_split) {
  return ts_verify_attn_workspace_size(n_part, Tq, Hq, Hkv, d, n_split);
}

int ts_verify_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t s_head, int64_t s_pos,
                   int32_t n_ctx, int32_t T, const int32_t* parent, int32_t Hq, int32_t Hkv, int32_t d,
                   float scale, float* out, int32_t n_split, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "ts_verify_attn";
  int rc = check_attention(who, q, k, v, out, s_head, s_pos, n_ctx, T, Hq, Hkv, d, scale, n_split);
  if (rc) return rc;
  if (!parent) return fail(TS_EINVAL, "%s: parent is null", who);
  uint64_t anc[2 * TS_MAX_TREE];
  char why[160];
  if (!build_masks(parent, T, anc, why, sizeof(why))) return fail(TS_EINVAL, "%s: %s", who, why);
  return run_attention(who, q, k, v, s_head, s_pos, n_ctx, T, anc, Hq, Hkv, d, scale, out, nullptr, n_split, ws,
                       ws_bytes, stream);
}

int ts_verify_attn_scored(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t s_head, int64_t s_pos,
                          int32_t n_ctx, int32_t T, const int32_t* parent, int32_t Hq, int32_t Hkv, int32_t d,
                          float scale, float* out, float* scores, int32_t n_split, void* ws, size_t ws_bytes,
                          void* stream) {
  const char* who = "ts_verify_attn_scored";
  int rc = check_attention(who, q, k, v, out, s_head, s_pos, n_ctx, T, Hq, Hkv, d, scale, n_split);
  if (rc) return rc;
  if (!parent) return fail(TS_EINVAL, "%s: parent is null", who);
  if (!scores) return fail(TS_EINVAL, "%s: scores is null", who);
  if (!aligned(scores, 4)) return fail(TS_EINVAL, "%s: scores must be 4-byte aligned", who);
  if (ts::attn_row_blocks(T, Hq, Hkv) != 1)
    return fail(TS_ENOTSUP, "%s: the %d query rows of a KV head ((Hq/Hkv)*T) exceed the 256 that one workgroup sums",
                who, (Hq / Hkv) * T);
  uint64_t anc[2 * TS_MAX_TREE];
  char why[160];
  if (!build_masks(parent, T, anc, why, sizeof(why))) return fail(TS_EINVAL, "%s: %s", who, why);
  return run_attention(who, q, k, v, s_head, s_pos, n_ctx, T, anc, Hq, Hkv, d, scale, out, scores, n_split, ws,
                       ws_bytes, stream);
}

int ts_draft_attn(const uint16_t* q, const uint16_t* k_part, const uint16_t* v_part, int64_t s_head,
                  int64_t s_pos, int32_t n_part, int32_t Tq, int32_t Hq, int32_t Hkv, int32_t d, float scale,
                  float* out, int32_t n_split, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "ts_draft_attn";
  int rc = check_attention(who, q, k_part, v_part, out, s_head, s_pos, n_part, Tq, Hq, Hkv, d, scale, n_split);
  if (rc) return rc;
  // The drafting tokens form a chain: token t sees tokens 0..t.
  uint64_t anc[2 * TS_MAX_TREE];
  for (int i = 0; i < TS_MAX_TREE; ++i) {   // token i sees tokens 0..i
    const bool in = i < Tq;
    anc[2 * i] = !in ? 0ull : (i >= 63 ? ~0ull : (1ull << (i + 1)) - 1);
    anc[2 * i + 1] = !in || i < 64 ? 0ull : (i == 127 ? ~0ull : (1ull << (i - 63)) - 1);
  }
  return run_attention(who, q, k_part, v_part, s_head, s_pos, n_part, Tq, anc, Hq, Hkv, d, scale, out, nullptr,
                       n_split, ws, ws_bytes, stream);
}

int32_t ts_partial_kv_rows(int32_t n_ctx, int32_t n_sink, int32_t budget, int32_t n_recent) {
  if (n_ctx < 0 || n_sink < 0 || budget < 0 || n_recent < 0) return -1;
  return partial_rows(n_ctx, n_sink, budget, n_recent).n_part;
}

size_t ts_partial_kv_select_workspace_size(int32_t n_ctx, int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                                           int32_t budget) {
  if (n_ctx < 0 || T < 1 || T > TS_MAX_TREE || Hq < 1 || Hkv < 1 || Hq % Hkv || (d != 64 && d != 128) || budget < 0)
    return 0;
  return ts::select_workspace_bytes(n_ctx, T, Hq, Hkv, d, budget);
}

}  // extern "C"

namespace {

// Shared by the two logit-pass entry points (top-p / min-p, or eta).
int run_penalty(const char* who, const float* logits, int32_t rows, int32_t V, const int32_t* window, int32_t W,
                int64_t window_stride, float penalty, float temperature, float top_p, float min_p, int eta_mode,
                float eta_eps, float eta_alpha, float* logits_out, uint8_t* keep, float* probs, const float* u,
                int32_t* token, void* ws, size_t ws_bytes, void* stream) {
  if (!logits || !logits_out) return fail(TS_EINVAL, "%s: null logits pointer", who);
  if (rows < 1) return fail(TS_EINVAL, "%s: rows=%d must be >= 1", who, rows);
  if (V < 1) return fail(TS_EINVAL, "%s: V=%d must be >= 1", who, V);
  if (V > 262144) return fail(TS_ENOTSUP, "%s: V=%d exceeds 262144", who, V);
  if (W < 0) return fail(TS_EINVAL, "%s: W=%d is negative", who, W);
  if (W > 0 && !window) return fail(TS_EINVAL, "%s: window is null with W=%d", who, W);
  if (window_stride < 0 || (window_stride > 0 && window_stride < W))
    return fail(TS_EINVAL, "%s: window_stride=%lld must be 0 (shared) or >= W", who, (long long)window_stride);
  if (!(penalty > 0.f) || std::isinf(penalty)) return fail(TS_EINVAL, "%s: penalty must be finite and > 0", who);
  if (!(temperature > 0.f) || std::isinf(temperature)) return fail(TS_EINVAL, "%s: temperature must be finite and > 0", who);
  if (token && !u) return fail(TS_EINVAL, "%s: token output needs u", who);
  if (!aligned(logits, 4) || !aligned(logits_out, 4) || (probs && !aligned(probs, 4)) || (u && !aligned(u, 4)) ||
      (token && !aligned(token, 4)) || (W > 0 && !aligned(window, 4)))
    return fail(TS_EINVAL, "%s: float and int32 arrays must be 4-byte aligned", who);
  const size_t need = ts::penalty_workspace_bytes(rows, V);
  if (ws_bytes < need) return fail(TS_EWORKSPACE, "%s: workspace of %zu bytes, need %zu", who, ws_bytes, need);
  if (need > 0 && (!ws || !aligned(ws, 256))) return fail(TS_EINVAL, "%s: workspace must be non-null and 256-byte aligned", who);

  ts::PenaltyParams p;
  std::memset(&p, 0, sizeof(p));
  p.logits = logits;
  p.logits_out = logits_out;
  p.window = window;
  p.window_stride = window_stride;
  p.rows = rows;
  p.V = V;
  p.W = W;
  p.penalty = penalty;
  p.temperature = temperature;
  p.inv_temperature = 1.0f / temperature;
  p.top_p = top_p;
  p.min_p = min_p;
  p.eta_mode = eta_mode;
  p.eta_eps = eta_eps;
  p.eta_alpha = eta_alpha;
  p.keep = keep;
  p.probs = probs;
  p.u = u;
  p.token = token;
  p.ws = ws;
  const hipError_t e = ts::launch_penalty(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TS_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

// Shared by both selection entry points: q == nullptr means the scores are
// given (scores_in) and no query pass runs.
int run_select(const char* who, const uint16_t* q, int32_t T, int32_t Hq, const float* scores_in,
               const uint16_t* k, const uint16_t* v, int64_t s_head, int64_t s_pos, int32_t n_ctx, int32_t Hkv,
               int32_t d, int32_t n_sink, int32_t budget, int32_t n_recent, int32_t* sel_idx, uint16_t* k_part,
               uint16_t* v_part, int64_t sp_head, int64_t sp_pos, int32_t* n_part_out, float* scores_out, void* ws,
               size_t ws_bytes, void* stream) {
  const bool given = q == nullptr;
  if (given ? !scores_in : false) return fail(TS_EINVAL, "%s: scores is null", who);
  if (!k || !v || !sel_idx || !k_part || !v_part || !n_part_out)
    return fail(TS_EINVAL, "%s: null pointer argument", who);
  if (d != 64 && d != 128) return fail(TS_ENOTSUP, "%s: head dim %d not supported (64 or 128)", who, d);
  if (!given) {
    if (T < 1) return fail(TS_EINVAL, "%s: need at least one query (got %d)", who, T);
    if (T > TS_MAX_TREE) return fail(TS_ENOTSUP, "%s: %d queries exceed the %d limit", who, T, TS_MAX_TREE);
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
      return fail(TS_EINVAL, "%s: Hq=%d must be a positive multiple of Hkv=%d", who, Hq, Hkv);
  } else if (Hkv < 1) {
    return fail(TS_EINVAL, "%s: Hkv=%d must be positive", who, Hkv);
  }
  if (Hkv > 65535) return fail(TS_ENOTSUP, "%s: Hkv=%d too large", who, Hkv);
  if (n_ctx < 0 || n_sink < 0 || budget < 0 || n_recent < 0)
    return fail(TS_EINVAL, "%s: n_ctx, n_sink, budget and n_recent must be >= 0", who);
  if (s_pos < d || s_pos % 8 || s_head < 0 || s_head % 8 || (Hkv > 1 && s_head == 0))
    return fail(TS_EINVAL, "%s: bad cache strides (s_head=%lld, s_pos=%lld)", who, (long long)s_head, (long long)s_pos);
  if (sp_pos < d || sp_pos % 8 || sp_head < 0 || sp_head % 8)
    return fail(TS_EINVAL, "%s: bad partial-cache strides (sp_head=%lld, sp_pos=%lld)", who, (long long)sp_head,
                (long long)sp_pos);
  if ((q && !aligned(q, 16)) || !aligned(k, 16) || !aligned(v, 16) || !aligned(k_part, 16) || !aligned(v_part, 16) ||
      !aligned(sel_idx, 4) || (scores_out && !aligned(scores_out, 4)) || (scores_in && !aligned(scores_in, 4)))
    return fail(TS_EINVAL, "%s: tensors must be 16-byte aligned (indices and scores 4-byte)", who);

  const PartialRows pr = partial_rows(n_ctx, n_sink, budget, n_recent);
  const int32_t cand_lo = pr.cand_lo, cand_hi = pr.cand_hi, b_eff = pr.b_eff, n_part = pr.n_part;
  if (Hkv > 1 && sp_head < (int64_t)n_part * sp_pos)
    return fail(TS_EINVAL, "%s: partial heads overlap (sp_head=%lld < n_part*sp_pos)", who, (long long)sp_head);

  const size_t need = given ? ts::select_passes_workspace_bytes(n_ctx, Hkv)
                            : ts::select_workspace_bytes(n_ctx, T, Hq, Hkv, d, budget);
  if (ws_bytes < need) return fail(TS_EWORKSPACE, "%s: workspace of %zu bytes, need %zu", who, ws_bytes, need);
  if (need > 0 && (!ws || !aligned(ws, 256))) return fail(TS_EINVAL, "%s: workspace must be non-null and 256-byte aligned", who);

  ts::SelectParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.v = v;
  p.s_head = s_head;
  p.s_pos = s_pos;
  p.n_ctx = n_ctx;
  p.T = T;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.d = d;
  p.n_sink = n_sink;
  p.budget = budget;
  p.n_recent = n_recent;
  p.cand_lo = cand_lo;
  p.cand_hi = cand_hi;
  p.b_eff = b_eff;
  p.n_part = n_part;
  p.sel_idx = sel_idx;
  p.k_part = k_part;
  p.v_part = v_part;
  p.sp_head = sp_head;
  p.sp_pos = sp_pos;
  char* w = static_cast<char*>(ws);
  if (given) {
    // read-only in this mode: only the query pass writes scores
    p.scores = const_cast<float*>(scores_in);
    p.scores_given = 1;
  } else {
    // workspace: scores (if not user-provided) | selection passes
    const size_t score_bytes = ((size_t)Hkv * n_ctx * sizeof(float) + 255) / 256 * 256;
    p.scores = scores_out ? scores_out : reinterpret_cast<float*>(w);
    w += score_bytes;
  }
  p.sel_ws = reinterpret_cast<int32_t*>(w);
  *n_part_out = n_part;
  const hipError_t e = ts::launch_select(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TS_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int ts_partial_kv_select(const uint16_t* q, int32_t T, const uint16_t* k, const uint16_t* v, int64_t s_head,
                         int64_t s_pos, int32_t n_ctx, int32_t Hq, int32_t Hkv, int32_t d, int32_t n_sink,
                         int32_t budget, int32_t n_recent, int32_t* sel_idx, uint16_t* k_part, uint16_t* v_part,
                         int64_t sp_head, int64_t sp_pos, int32_t* n_part_out, float* scores, void* ws,
                         size_t ws_bytes, void* stream) {
  const char* who = "ts_partial_kv_select";
  if (!q) return fail(TS_EINVAL, "%s: q is null", who);
  return run_select(who, q, T, Hq, nullptr, k, v, s_head, s_pos, n_ctx, Hkv, d, n_sink, budget, n_recent, sel_idx,
                    k_part, v_part, sp_head, sp_pos, n_part_out, scores, ws, ws_bytes, stream);
}

size_t ts_partial_kv_select_scored_workspace_size(int32_t n_ctx, int32_t Hkv, int32_t d, int32_t budget) {
  if (n_ctx < 0 || Hkv < 1 || (d != 64 && d != 128) || budget < 0) return 0;
  return ts::select_passes_workspace_bytes(n_ctx, Hkv);
}

int ts_partial_kv_select_scored(const float* scores, const uint16_t* k, const uint16_t* v, int64_t s_head,
                                int64_t s_pos, int32_t n_ctx, int32_t Hkv, int32_t d, int32_t n_sink, int32_t budget,
                                int32_t n_recent, int32_t* sel_idx, uint16_t* k_part, uint16_t* v_part,
                                int64_t sp_head, int64_t sp_pos, int32_t* n_part_out, void* ws, size_t ws_bytes,
                                void* stream) {
  return run_select("ts_partial_kv_select_scored", nullptr, 0, 0, scores, k, v, s_head, s_pos, n_ctx, Hkv, d, n_sink,
                    budget, n_recent, sel_idx, k_part, v_part, sp_head, sp_pos, n_part_out, nullptr, ws, ws_bytes,
                    stream);
}

size_t ts_penalty_sample_workspace_size(int32_t rows, int32_t V) {
  if (rows < 1 || V < 1) return 0;
  return ts::penalty_workspace_bytes(rows, V);
}

int ts_penalty_sample(const float* logits, int32_t rows, int32_t V, const int32_t* window, int32_t W,
                      int64_t window_stride, float penalty, float temperature, float top_p, float min_p,
                      float* logits_out, uint8_t* keep, float* probs, const float* u, int32_t* token, void* ws,
                      size_t ws_bytes, void* stream) {
  const char* who = "ts_penalty_sample";
  if (!(top_p >= 0.f && top_p <= 1.f)) return fail(TS_EINVAL, "%s: top_p must lie in [0, 1]", who);
  if (!(min_p >= 0.f && min_p <= 1.f)) return fail(TS_EINVAL, "%s: min_p must lie in [0, 1]", who);
  return run_penalty(who, logits, rows, V, window, W, window_stride, penalty, temperature, top_p, min_p, 0, 0.f, 0.f,
                     logits_out, keep, probs, u, token, ws, ws_bytes, stream);
}

int ts_penalty_sample_eta(const float* logits, int32_t rows, int32_t V, const int32_t* window, int32_t W,
                          int64_t window_stride, float penalty, float temperature, float epsilon, float alpha,
                          float* logits_out, uint8_t* keep, float* probs, const float* u, int32_t* token, void* ws,
                          size_t ws_bytes, void* stream) {
  const char* who = "ts_penalty_sample_eta";
  if (!(epsilon > 0.f && epsilon <= 1.f)) return fail(TS_EINVAL, "%s: epsilon must lie in (0, 1]", who);
  if (!(alpha >= 0.f) || std::isinf(alpha)) return fail(TS_EINVAL, "%s: alpha must be finite and >= 0", who);
  return run_penalty(who, logits, rows, V, window, W, window_stride, penalty, temperature, 1.f, 0.f, 1, epsilon,
                     alpha, logits_out, keep, probs, u, token, ws, ws_bytes, stream);
}

int ts_tree_accept(const int32_t* parent, int32_t T, const int32_t* node_token, const int32_t* target,
                   int32_t* result, void* stream) {
  const char* who = "ts_tree_accept";
  if (!parent || !node_token || !target || !result) return fail(TS_EINVAL, "%s: null pointer argument", who);
  if (T < 1) return fail(TS_EINVAL, "%s: need at least one node (got %d)", who, T);
  if (T > TS_MAX_TREE) return fail(TS_ENOTSUP, "%s: %d nodes exceed the %d-node limit", who, T, TS_MAX_TREE);
  if (!aligned(node_token, 4) || !aligned(target, 4) || !aligned(result, 4))
    return fail(TS_EINVAL, "%s: token and result arrays must be 4-byte aligned", who);
  ts::AcceptParams p;
  std::memset(&p, 0, sizeof(p));
  char why[160];
  if (!build_masks(parent, T, p.anc, why, sizeof(why))) return fail(TS_EINVAL, "%s: %s", who, why);
  for (int i = 0; i < T; ++i) p.parent[i] = parent[i];
  p.node_token = node_token;
  p.target = target;
  p.result = result;
  p.T = T;
  const hipError_t e = ts::launch_accept(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TS_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

int ts_kv_commit(const int32_t* result, int32_t T, uint16_t* k, uint16_t* v, int64_t s_layer, int64_t s_head,
                 int64_t s_pos, int32_t layers, int32_t Hkv, int32_t d, int32_t n_ctx, uint16_t* k_part,
                 uint16_t* v_part, int64_t sp_layer, int64_t sp_head, int64_t sp_pos, int32_t n_part,
                 int32_t part_rows, void* stream) {
  const char* who = "ts_kv_commit";
  if (!result || !k || !v) return fail(TS_EINVAL, "%s: null pointer argument", who);
  if (T < 1) return fail(TS_EINVAL, "%s: need at least one node (got %d)", who, T);
  if (T > TS_MAX_TREE) return fail(TS_ENOTSUP, "%s: %d nodes exceed the %d-node limit", who, T, TS_MAX_TREE);
  if (d != 64 && d != 128) return fail(TS_ENOTSUP, "%s: head dim %d not supported (64 or 128)", who, d);
  if (layers < 1 || layers > 65535 || Hkv < 1 || Hkv > 65535)
    return fail(TS_EINVAL, "%s: layers=%d and Hkv=%d must lie in [1, 65535]", who, layers, Hkv);
  if (n_ctx < 0) return fail(TS_EINVAL, "%s: n_ctx=%d is negative", who, n_ctx);
  if ((int64_t)n_ctx + T > (int64_t)INT32_MAX) return fail(TS_EINVAL, "%s: cache rows overflow int32", who);
  if (s_pos < d || s_pos % 8 || s_head < 0 || s_head % 8 || s_layer < 0 || s_layer % 8 || (Hkv > 1 && s_head == 0) ||
      (layers > 1 && s_layer == 0))
    return fail(TS_EINVAL, "%s: bad cache strides (s_layer=%lld, s_head=%lld, s_pos=%lld)", who, (long long)s_layer,
                (long long)s_head, (long long)s_pos);
  if (!aligned(result, 4) || !aligned(k, 16) || !aligned(v, 16))
    return fail(TS_EINVAL, "%s: k and v must be 16-byte aligned, result 4-byte", who);
  if ((k_part == nullptr) != (v_part == nullptr)) return fail(TS_EINVAL, "%s: give both k_part and v_part or neither", who);
  if (k_part) {
    if (sp_pos < d || sp_pos % 8 || sp_head < 0 || sp_head % 8 || sp_layer < 0 || sp_layer % 8 ||
        (Hkv > 1 && sp_head == 0) || (layers > 1 && sp_layer == 0))
      return fail(TS_EINVAL, "%s: bad partial-cache strides", who);
    if (!aligned(k_part, 16) || !aligned(v_part, 16)) return fail(TS_EINVAL, "%s: partial caches must be 16-byte aligned", who);
    if (n_part < 0 || part_rows < 0 || (int64_t)n_part + T > (int64_t)part_rows)
      return fail(TS_EINVAL, "%s: n_part=%d + T=%d rows exceed the partial cache's %d rows", who, n_part, T, part_rows);
  }
  ts::CommitParams p;
  std::memset(&p, 0, sizeof(p));
  p.result = result;
  p.k = k;
  p.v = v;
  p.s_layer = s_layer;
  p.s_head = s_head;
  p.s_pos = s_pos;
  p.layers = layers;
  p.Hkv = Hkv;
  p.d = d;
  p.n_ctx = n_ctx;
  p.T = T;
  p.k_part = k_part;
  p.v_part = v_part;
  p.sp_layer = sp_layer;
  p.sp_head = sp_head;
  p.sp_pos = sp_pos;
  p.n_part = n_part;
  const hipError_t e = ts::launch_commit(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TS_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

int ts_ngram_tree(const int32_t* window, int32_t W, int32_t k, uint64_t seed, const int32_t* head_cand,
                  int32_t levels, int32_t T_max, int32_t* parent, int32_t* node_token, int32_t* info, void* stream) {
  const char* who = "ts_ngram_tree";
  if (!window || !parent || !node_token || !info) return fail(TS_EINVAL, "%s: null pointer argument", who);
  if (W < 1) return fail(TS_EINVAL, "%s: the window needs at least the root token (W=%d)", who, W);
  if (W > ts::NG_MAX_WINDOW) return fail(TS_ENOTSUP, "%s: W=%d exceeds %d tokens", who, W, ts::NG_MAX_WINDOW);
  if (k < 0) return fail(TS_EINVAL, "%s: k=%d is negative", who, k);
  if (levels < 0 || levels > 3) return fail(TS_EINVAL, "%s: levels=%d must lie in [0, 3]", who, levels);
  if (levels > 0 && !head_cand) return fail(TS_EINVAL, "%s: head_cand is null with %d levels", who, levels);
  if (T_max < 1 || T_max > TS_MAX_TREE) return fail(TS_EINVAL, "%s: T_max=%d must lie in [1, %d]", who, T_max, TS_MAX_TREE);
  if (!aligned(window, 4) || !aligned(parent, 4) || !aligned(node_token, 4) || !aligned(info, 4) ||
      (head_cand && !aligned(head_cand, 4)))
    return fail(TS_EINVAL, "%s: int32 arrays must be 4-byte aligned", who);
  ts::NgramParams p;
  std::memset(&p, 0, sizeof(p));
  p.window = window;
  p.head = levels > 0 ? head_cand : nullptr;
  p.parent = parent;
  p.node_token = node_token;
  p.info = info;
  p.seed = seed;
  p.W = W;
  p.k = k;
  p.levels = levels;
  p.T_max = T_max;
  const hipError_t e = ts::launch_ngram_tree(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TS_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

}  // extern "C"
