// C-ABI entry points of librelattn: argument validation (host only), plan
// selection and launch.  The operation is defined in include/relattn.h.
#include "relattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "relattn_internal.h"

namespace {

using relattn::FwdParams;
using relattn::LaunchCfg;
using relattn::RelMode;
using relattn::T5Buckets;

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

constexpr size_t kMaxLdsBytes = 160 * 1024;  // LDS per workgroup on gfx950
// compute units of an MI355X; only the launch-shape heuristic uses it (the
// plan is made on the host, without a device)
constexpr int64_t kNumCUs = 256;
constexpr int64_t kMaxSeq = int64_t(1) << 30;

size_t elem_size(int dtype) { return dtype == RELATTN_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t numel(const relattn_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

// Shape-independent checks of a strided view with `ndim` dims, innermost
// contiguous; `vec_rows`: rows are read with 16-byte vector loads.
int check_view(const relattn_tensor* t, const char* name, int ndim, bool vec_rows) {
  if (!t) return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (t->ndim != ndim)
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s must have %d dims, got %d", name, ndim,
                t->ndim);
  if (t->dtype != RELATTN_F32 && t->dtype != RELATTN_BF16)
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s has unknown dtype %d", name, t->dtype);
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s shape[%d] < 0", name, i);
    if (t->stride[i] < 0)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s stride[%d] < 0", name, i);
  }
  if (numel(t) == 0) return RELATTN_OK;
  if (!t->data) return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s data is NULL", name);
  if (t->stride[ndim - 1] != 1)
    return fail(RELATTN_ERR_UNSUPPORTED, "%s: innermost dimension must be contiguous", name);
  if (vec_rows) {
    const size_t es = elem_size(t->dtype);
    if (!aligned16(t->data))
      return fail(RELATTN_ERR_UNSUPPORTED, "%s: data pointer is not 16-byte aligned", name);
    for (int i = 0; i + 1 < ndim; ++i)
      if ((t->stride[i] * es) % 16 != 0)
        return fail(RELATTN_ERR_UNSUPPORTED, "%s: stride[%d] is not a multiple of 16 bytes",
                    name, i);
  }
  return RELATTN_OK;
}

// ---- T5 bucket thresholds, exact ------------------------------------------
// floor(nlog * ln(a/ex) / ln(D/ex)) >= t  <=>  a^nlog * ex^t >= D^t * ex^nlog,
// evaluated with arbitrary-precision unsigned integers.
struct Big {
  std::vector<uint32_t> w{1u};
  void mul(uint32_t m) {
    uint64_t carry = 0;
    for (auto& d : w) {
      const uint64_t t = uint64_t(d) * m + carry;
      d = uint32_t(t);
      carry = t >> 32;
    }
    if (carry) w.push_back(uint32_t(carry));
  }
};

int cmp_big(const Big& x, const Big& y) {
  size_t nx = x.w.size(), ny = y.w.size();
  while (nx > 1 && x.w[nx - 1] == 0) --nx;
  while (ny > 1 && y.w[ny - 1] == 0) --ny;
  if (nx != ny) return nx < ny ? -1 : 1;
  for (size_t i = nx; i-- > 0;)
    if (x.w[i] != y.w[i]) return x.w[i] < y.w[i] ? -1 : 1;
  return 0;
}

bool log_bucket_at_least(uint32_t a, uint32_t ex, uint32_t D, int nlog, int t) {
  Big lhs, rhs;
  for (int i = 0; i < nlog; ++i) lhs.mul(a);
  for (int i = 0; i < t; ++i) lhs.mul(ex);
  for (int i = 0; i < t; ++i) rhs.mul(D);
  for (int i = 0; i < nlog; ++i) rhs.mul(ex);
  return cmp_big(lhs, rhs) >= 0;
}

int check_t5(const relattn_t5_params* t5, T5Buckets* out) {
  const int nb = t5->num_buckets;
  const bool bidir = t5->bidirectional != 0;
  if (nb < 2) return fail(RELATTN_ERR_INVALID_ARGUMENT, "num_buckets must be >= 2");
  if (bidir && (nb % 2 != 0 || nb < 4))
    return fail(RELATTN_ERR_INVALID_ARGUMENT,
                "bidirectional bucketing needs an even num_buckets >= 4");
  const int half = bidir ? nb / 2 : nb;
  const int exact = half / 2;
  const int nlog = half - exact;
  if (t5->max_distance <= exact)
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "max_distance (%d) must exceed B_exact (%d)",
                t5->max_distance, exact);
  if (nlog - 1 > relattn::kMaxT5Thresholds)
    return fail(RELATTN_ERR_UNSUPPORTED, "num_buckets too large (at most %d log buckets)",
                relattn::kMaxT5Thresholds + 1);
  if (!out) return RELATTN_OK;
  // Memoised per thread: the thresholds depend only on (nb, D, bidir).
  thread_local int c_nb = -1, c_d = -1, c_bi = -1;
  thread_local T5Buckets c_tb;
  if (c_nb == nb && c_d == t5->max_distance && c_bi == (int)bidir) {
    *out = c_tb;
    return RELATTN_OK;
  }
  T5Buckets tb = {};
  tb.nb = nb;
  tb.half = half;
  tb.exact = exact;
  tb.nlog = nlog;
  tb.bidir = bidir ? 1 : 0;
  const uint32_t D = (uint32_t)t5->max_distance, ex = (uint32_t)exact;
  for (int t = 1; t < nlog; ++t) {
    uint32_t lo = ex, hi = D;  // the condition holds at a = D
    while (lo < hi) {
      const uint32_t mid = lo + (hi - lo) / 2;
      if (log_bucket_at_least(mid, ex, D, nlog, t)) hi = mid;
      else lo = mid + 1;
    }
    tb.thr[t - 1] = (int32_t)lo;
  }
  c_nb = nb;
  c_d = t5->max_distance;
  c_bi = (int)bidir;
  c_tb = tb;
  *out = tb;
  return RELATTN_OK;
}

struct Plan {
  bool empty = false;
  bool bf16 = false;
  int d = 0;
  LaunchCfg cfg{2, 64, 2, relattn::kWvResident};
  RelMode mode = relattn::kRelNone;
  bool has_wk = false, has_wv = false;
  FwdParams p{};
};

int check_table(const relattn_tensor* t, const char* name, const relattn_tensor* q,
                int clip_k) {
  int st = check_view(t, name, 3, true);
  if (st) return st;
  if (t->dtype != q->dtype)
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s dtype differs from q", name);
  const int64_t H = q->shape[1], d = q->shape[3];
  if (!(t->shape[0] == H || t->shape[0] == 1))
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s: shape[0] must be H (%lld) or 1", name,
                (long long)H);
  if (t->shape[1] != 2 * (int64_t)clip_k + 1)
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s: shape[1] must be 2*clip_k+1 = %lld", name,
                (long long)(2 * (int64_t)clip_k + 1));
  if (t->shape[2] != d)
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s: shape[2] must equal d = %lld", name,
                (long long)d);
  return RELATTN_OK;
}

int make_plan(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
              const relattn_tensor* wK, const relattn_tensor* wV,
              const relattn_tensor* t5_bias, const relattn_t5_params* t5, int32_t clip_k,
              float scale, const relattn_mask* mask, const relattn_tensor* out, Plan* plan,
              bool want_t5_table, const relattn_tensor* ob = nullptr, int32_t ob_window = 0,
              const relattn_tensor* xl_u = nullptr, const relattn_tensor* xl_v = nullptr,
              int32_t grid_m = 0, const relattn_tensor* labels = nullptr) {
  int st;
  if ((st = check_view(q, "q", 4, true))) return st;
  if ((st = check_view(k, "k", 4, true))) return st;
  if ((st = check_view(v, "v", 4, true))) return st;
  if ((st = check_view(out, "out", 4, true))) return st;
  const relattn_tensor* others[3] = {k, v, out};
  const char* names[3] = {"k", "v", "out"};
  for (int t = 0; t < 3; ++t) {
    if (others[t]->dtype != q->dtype)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s dtype differs from q", names[t]);
    for (int i = 0; i < 4; ++i)
      if (others[t]->shape[i] != q->shape[i])
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s shape differs from q in dim %d",
                    names[t], i);
  }
  const int64_t B = q->shape[0], H = q->shape[1], n = q->shape[2], d = q->shape[3];
  if (!(d == 16 || d == 32 || d == 64 || d == 128))
    return fail(RELATTN_ERR_UNSUPPORTED, "head size d = %lld is not one of 16, 32, 64, 128",
                (long long)d);
  if (n > kMaxSeq)
    return fail(RELATTN_ERR_UNSUPPORTED, "sequence length %lld exceeds 2^30", (long long)n);
  if (std::isnan(scale) || std::isinf(scale))
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "scale must be finite");

  const bool is_t5 = t5_bias != nullptr || t5 != nullptr;
  const bool is_ob = ob != nullptr;  // scalar bias by clipped offset, 2-D offset or label
  const bool is_lab = labels != nullptr;  // ... by a per-pair label (or key/value tables)
  if (is_lab && (grid_m > 0 || is_t5 || (!is_ob && !wK && !wV)))
    return fail(RELATTN_ERR_INVALID_ARGUMENT,
                "edge labels take a bias table or key/value tables by label");
  if (is_lab) {
    // [B, n, n] uint8 labels, rows read in whole 16-byte chunks
    if (labels->ndim != 3)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels must have 3 dims, got %d", labels->ndim);
    if (labels->dtype != RELATTN_U8)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels must be U8");
    if (labels->shape[0] != q->shape[0] || labels->shape[1] != q->shape[2] ||
        labels->shape[2] != q->shape[2])
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels must be [B, n, n]");
    for (int i = 0; i < 3; ++i)
      if (labels->stride[i] < 0)
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels stride[%d] < 0", i);
    if (numel(labels) > 0) {
      const int64_t n16 = (q->shape[2] + 15) / 16 * 16;
      if (!labels->data) return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels data is NULL");
      if (labels->stride[2] != 1)
        return fail(RELATTN_ERR_UNSUPPORTED, "labels: innermost dimension must be contiguous");
      if (!aligned16(labels->data))
        return fail(RELATTN_ERR_UNSUPPORTED, "labels: data pointer is not 16-byte aligned");
      if (labels->stride[1] % 16 != 0 || labels->stride[0] % 16 != 0)
        return fail(RELATTN_ERR_UNSUPPORTED, "labels: strides must be multiples of 16 bytes");
      if (labels->stride[1] < n16)
        return fail(RELATTN_ERR_UNSUPPORTED,
                    "labels: row stride %lld is below n rounded up to 16 (%lld)",
                    (long long)labels->stride[1], (long long)n16);
    }
  }
  const bool is_graph = is_lab && !is_ob;  // Shaw tables indexed by label
  if ((t5_bias == nullptr) != (t5 == nullptr))
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "t5_bias and t5 params must be given together");
  if (is_t5 && (wK || wV))
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "T5 bias excludes the wK/wV tables");
  if (is_ob && (wK || wV || is_t5))
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "an offset bias excludes the other tables");
  if (!is_t5 && !is_ob && clip_k < 0)
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "clip_k must be >= 0");
  if (!is_t5 && !is_ob && (int64_t)clip_k > kMaxSeq)
    return fail(RELATTN_ERR_UNSUPPORTED, "clip_k exceeds 2^30");
  if (is_ob) {
    if ((st = check_view(ob, "bias", 2, false))) return st;
    if (ob->dtype != RELATTN_F32) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias must be F32");
    if (ob_window < 0) return fail(RELATTN_ERR_INVALID_ARGUMENT, "window must be >= 0");
    if ((int64_t)ob_window > kMaxSeq) return fail(RELATTN_ERR_UNSUPPORTED, "window exceeds 2^30");
    if (!(ob->shape[0] == q->shape[1] || ob->shape[0] == 1))
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias: shape[0] must be H (%lld) or 1",
                  (long long)q->shape[1]);
    if (grid_m > 0) {
      // 2-D window of M x M raster tokens, table by flattened 2-D offset
      if (grid_m > 2048)
        return fail(RELATTN_ERR_UNSUPPORTED, "window side M = %d exceeds 2048", grid_m);
      if (q->shape[2] != (int64_t)grid_m * grid_m)
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "n (%lld) must be M*M = %lld",
                    (long long)q->shape[2], (long long)grid_m * grid_m);
      if (ob->shape[1] != (int64_t)(2 * grid_m - 1) * (2 * grid_m - 1))
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias: shape[1] must be (2M-1)^2 = %lld",
                    (long long)(2 * grid_m - 1) * (2 * grid_m - 1));
      if (mask && mask->causal)
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "a 2-D window bias takes no causal mask");
    } else if (is_lab) {
      if (ob->shape[1] < 1 || ob->shape[1] > 256)
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias: shape[1] (labels) must be in [1, 256]");
    } else if (ob->shape[1] != 2 * (int64_t)ob_window + 1) {
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias: shape[1] must be 2*window+1 = %lld",
                  (long long)(2 * (int64_t)ob_window + 1));
    }
  }
  const bool is_xl = xl_u != nullptr || xl_v != nullptr;
  if (is_xl) {
    // Transformer-XL: wK is the position table R (read by i - j), u and v the
    // global biases; no value table, no scalar bias
    if (!xl_u || !xl_v || !wK)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "R, u and v must be given together");
    if (wV || is_t5 || is_ob)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "Transformer-XL logits exclude the other tables");
    const relattn_tensor* uv[2] = {xl_u, xl_v};
    const char* nm[2] = {"u", "v"};
    for (int t = 0; t < 2; ++t) {
      if ((st = check_view(uv[t], nm[t], 2, true))) return st;
      if (uv[t]->dtype != q->dtype)
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s dtype differs from q", nm[t]);
      if (!(uv[t]->shape[0] == q->shape[1] || uv[t]->shape[0] == 1) ||
          uv[t]->shape[1] != q->shape[3])
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s must be [H or 1, d]", nm[t]);
    }
  }
  int64_t n_labels = 0;  // graph mode: rows of the key/value tables
  if (is_graph) {
    const relattn_tensor* tabs[2] = {wK, wV};
    const char* nm[2] = {"wK", "wV"};
    for (int t = 0; t < 2; ++t) {
      if (!tabs[t]) continue;
      if ((st = check_view(tabs[t], nm[t], 3, true))) return st;
      if (tabs[t]->dtype != q->dtype)
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s dtype differs from q", nm[t]);
      if (!(tabs[t]->shape[0] == H || tabs[t]->shape[0] == 1) || tabs[t]->shape[2] != d)
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s must be [H or 1, NL, d]", nm[t]);
      if (tabs[t]->shape[1] < 1 || tabs[t]->shape[1] > 256)
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s: NL = shape[1] must be in [1, 256]", nm[t]);
      if (n_labels && tabs[t]->shape[1] != n_labels)
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "wK and wV must have the same NL");
      n_labels = tabs[t]->shape[1];
    }
  } else {
    if (wK && (st = check_table(wK, is_xl ? "R" : "wK", q, clip_k))) return st;
    if (wV && (st = check_table(wV, "wV", q, clip_k))) return st;
  }
  T5Buckets tb = {};
  if (is_t5) {
    if ((st = check_view(t5_bias, "t5_bias", 2, false))) return st;
    if (t5_bias->dtype != RELATTN_F32)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "t5_bias must be F32");
    if (t5_bias->shape[0] != t5->num_buckets || t5_bias->shape[1] != H)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "t5_bias must be [num_buckets, H]");
    if ((st = check_t5(t5, want_t5_table ? &tb : nullptr))) return st;
  }
  if (mask && mask->key_lens && (reinterpret_cast<uintptr_t>(mask->key_lens) & 3u))
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "key_lens is not 4-byte aligned");

  Plan& P = *plan;
  P.bf16 = q->dtype == RELATTN_BF16;
  P.d = (int)d;
  P.mode = is_graph ? relattn::kRelGraph
          : is_lab ? relattn::kRelLabel
                  : (is_xl && (d <= 64 || (q->dtype == RELATTN_BF16 && d == 128))) ? relattn::kRelXL
                  : (is_ob && grid_m > 0) ? relattn::kRelGrid
                  : (is_t5 || is_ob) ? relattn::kRelT5
                                     : ((wK || wV) ? relattn::kRelShaw : relattn::kRelNone);
  P.has_wk = wK != nullptr;
  P.has_wv = wV != nullptr;
  P.empty = (B == 0 || H == 0 || n == 0);
  if (P.empty) return RELATTN_OK;

  FwdParams& p = P.p;
  p.B = (int32_t)B;
  p.H = (int32_t)H;
  p.n = (int32_t)n;
  p.causal = (mask && mask->causal) ? 1 : 0;
  p.key_lens = mask ? mask->key_lens : nullptr;
  p.clip = (is_t5 || is_ob) ? 0 : clip_k;
  const bool causal = p.causal != 0;
  // Label rows any query can reach: offsets j - i lie in [-(n-1), n-1], or in
  // [-(n-1), 0] under the causal mask.
  if (P.mode == relattn::kRelGraph) {
    p.r_lo = 0;
    p.nr = (int32_t)n_labels;
  } else if (P.mode == relattn::kRelShaw) {
    const int64_t c = clip_k;
    const int64_t r_lo = std::max<int64_t>(0, c - (n - 1));
    const int64_t r_hi = causal ? c : std::min<int64_t>(2 * c, c + n - 1);
    p.r_lo = (int32_t)r_lo;
    p.nr = (int32_t)(r_hi - r_lo + 1);
  } else {
    p.r_lo = 0;
    p.nr = 1;
  }
  p.t5_dist = is_t5 ? (int32_t)std::min<int64_t>(t5->max_distance, n - 1)
                    : ((is_ob && !is_lab) ? (int32_t)std::min<int64_t>(ob_window, n - 1) : 0);
  if (is_graph) {
    p.lab = static_cast<const uint8_t*>(labels->data);
    p.lab_sb = labels->stride[0];
    p.lab_sn = labels->stride[1];
  } else if (is_lab) {
    // the head's row of NL entries is loaded and indexed by each pair's label
    tb.nb = (int32_t)ob->shape[1];
    p.ob = 1;
    p.ob_lo = 0;
    p.lab = static_cast<const uint8_t*>(labels->data);
    p.lab_sb = labels->stride[0];
    p.lab_sn = labels->stride[1];
  } else if (is_ob && grid_m > 0) {
    // every offset is in the band (no end value); the (2M-1)^2 entries of the
    // head's row are loaded and indexed per key from the 2-D offset
    p.t5_dist = (int32_t)(n - 1);
    tb.nb = (2 * grid_m - 1) * (2 * grid_m - 1);
    p.ob = 1;
    p.ob_lo = 0;
    p.grid_m = grid_m;
    p.grid_inv = 1.f / (float)grid_m;
  } else if (is_ob) {
    // the table's entries for offsets -t5_dist .. t5_dist stand in for the
    // bucket column; offsets beyond them take the end entries, as buckets do
    tb.nb = 2 * p.t5_dist + 1;
    p.ob = 1;
    p.ob_lo = ob_window - p.t5_dist;
  }
  p.t5 = tb;
  const float s = scale > 0.f ? scale
                              : (is_t5 ? 1.f : 1.f / std::sqrt((float)d));
  p.scale_log2 = s * 1.4426950408889634f;

  // Workgroup shape: 32 query rows per wave, 64-key (bf16) or 32-key (fp32)
  // tiles, a 2- or 3-tile K/V ring and one of three places for the w^V rows.
  // Among the shapes whose LDS fits, take the one that keeps the most waves
  // of this grid resident per compute unit (two per SIMD for d <= 64, one
  // for d = 128, as the kernels are compiled); ties go to the earlier one.
  const int nb = is_t5 ? t5->num_buckets : (is_ob ? p.t5.nb : 0);  // entries staged
  // A window whose per-query rows (or per-head vector) alone exceed a
  // workgroup's LDS can never fit.  Rejecting it before any layout is sized
  // also keeps the layouts' 32-bit byte arithmetic far from overflow (rows of
  // 2^22 labels times 128 query rows would wrap).
  {
    constexpr int64_t kMaxEntries = (int64_t)(kMaxLdsBytes / 4);  // fp32 entries
    const int64_t win = (P.mode == relattn::kRelShaw || P.mode == relattn::kRelGraph)
                            ? (int64_t)p.nr
                            : 2 * (int64_t)p.t5_dist + 1;
    if (win > kMaxEntries || (int64_t)nb > kMaxEntries)
      return fail(RELATTN_ERR_UNSUPPORTED,
                  "a window of %lld offsets (%d staged entries) does not fit on chip",
                  (long long)win, nb);
  }
  auto lds_of = [&](const LaunchCfg& c) {
    return relattn::lds_bytes(P.bf16, P.d, c, P.mode, P.has_wk, P.has_wv, p.nr, p.t5_dist, nb);
  };
  std::vector<int> waves;
  std::vector<int> kblocks;
  if (P.bf16) {
    // four waves first: a workgroup then shares each K/V tile among 128
    // query rows (measured faster than two waves even when that leaves one
    // workgroup per compute unit, e.g. B32 H8 n128)
    waves = {4, 2, 1};
    // fused Transformer-XL: each wave reads its own table rows per tile, and
    // two two-wave workgroups per compute unit hide that latency better than
    // one four-wave workgroup (measured 33.8 vs 37.0 us on B8 H16 n512 d64)
    if (P.mode == relattn::kRelXL) waves = {2, 4, 1};
    kblocks = {64};
    // two waves per SIMD at d = 128 with 32-key tiles, except for the fused
    // Transformer-XL mode, whose table fragments spill there (it runs one wave
    // per SIMD with 64-key tiles)
    if (d == 128 && P.mode != relattn::kRelXL) kblocks.push_back(32);
  } else {
    kblocks = {32};
    if (n <= 32) waves = {1, 2};
    else waves = {2, 1};
  }
  // waves per CU the kernels' register budget allows (4 SIMDs; the same rule
  // as the kernels')
  auto vgpr_waves_per_cu = [&](int kblock, int waves) {
    if (d > 64) return 4 * ((P.bf16 && kblock == 32) ? 2 : 1);
    return 4 * ((P.bf16 && P.mode != relattn::kRelShaw && P.mode != relattn::kRelXL &&
                 P.mode != relattn::kRelGraph && (d <= 32 || waves == 4)) ? 3 : 2);
  };
  // a workgroup whose lower half of waves already covers every query row
  // would leave the rest idle (short windows, e.g. 7 x 7 = 49 tokens)
  {
    std::vector<int> keep;
    for (int w : waves)
      if (w == 1 || 32 * (w / 2) < n) keep.push_back(w);
    waves = keep;
  }
  bool found_lean = false;
  // Small windows of the 2-D window bias: the persistent window kernel
  // (a whole window is one key tile; items stream through two LDS slots)
  if (P.mode == relattn::kRelGrid &&
      relattn::window_grid_ok(P.bf16, P.d, (int)n, grid_m,
                              std::max({q->stride[2], k->stride[2], v->stride[2]}))) {
    P.cfg = LaunchCfg{2, 64, 1, relattn::kWvResident, 3};
    found_lean = true;
  }
  // The lean bf16 kernel serves the Shaw tables and plain attention at d = 64
  // whenever its resident tables and relative rows fit.  Among its shapes take
  // the one that keeps the most waves of this grid resident per compute unit
  // (two per SIMD); on a tie the four-wave shape (two workgroups per compute
  // unit drift apart in phase, so one's exponentials overlap the other's
  // products: measured 14.1 us against 16.3 us for one eight-wave workgroup on
  // the Transformer-big causal shape), then the deepest ring (a ring that
  // holds every tile of a workgroup requests them all at entry).
  if (!found_lean && relattn::lean_mode_ok(P.bf16, P.d, P.mode) && !is_xl) {
    const int kb = P.d == 64 ? 64 : 32;
    int64_t best_res = -1;
    int best_st = -1, best_w = -1;
    for (int w : {4, 8}) {
      if (w == 8 && n <= 128) continue;  // half the waves would hold no query row
      const int64_t wgs = B * H * ((n + 32 * w - 1) / (32 * w));
      const int64_t need = (wgs + kNumCUs - 1) / kNumCUs;
      const int64_t max_tiles = (n + kb - 1) / kb;  // tiles of the heaviest workgroup
      for (int st = (int)std::min<int64_t>(max_tiles, 8); st >= 1; --st) {
        if (st == 1 && max_tiles > 1) break;  // a ring needs two stages
        const LaunchCfg c{w, kb, st, relattn::kWvResident, 1};
        const size_t lds = relattn::lean_lds_bytes(P.d, c, P.mode, P.has_wk, P.has_wv, p.nr,
                                                   p.t5_dist, nb);
        if (lds > kMaxLdsBytes) continue;
        const int64_t fit = std::min<int64_t>(8 / w, (int64_t)(kMaxLdsBytes / lds));
        const int64_t resident = std::min(fit, need) * w;
        if (resident > best_res || (resident == best_res && w == best_w && st > best_st)) {
          best_res = resident;
          best_st = st;
          best_w = w;
          P.cfg = c;
        }
      }
    }
    if (best_res > 0) found_lean = true;
  }
  std::vector<LaunchCfg> order;
  for (int kb : kblocks)
    for (int w : waves)
      // two-tile rings first: measured as fast or faster than three on every
      // workload (headline 15.5 -> 15.0 us, long 291 -> 209 us, 2-D window
      // 33.3 -> 29.7 us, T5 and base within 2%); a third stage only takes LDS
      for (int st : {2, 3})
        for (int wm : {relattn::kWvResident, relattn::kWvRing, relattn::kWvChunked})
          order.push_back({w, kb, st, wm});
  bool found = found_lean;
  int64_t best = -1;
  for (const auto& c : order) {
    if (found_lean) break;
    const size_t lds = lds_of(c);
    if (lds > kMaxLdsBytes) continue;
    const int64_t wgs = B * H * ((n + 32 * c.waves - 1) / (32 * c.waves));
    const int64_t fit = std::min<int64_t>(vgpr_waves_per_cu(c.kblock, c.waves) / c.waves,
                                          lds ? (int64_t)(kMaxLdsBytes / lds) : 64);
    const int64_t need = (wgs + kNumCUs - 1) / kNumCUs;  // workgroups per CU in one round
    const int64_t resident = std::min(fit, need) * c.waves;
    if (resident > best) {
      best = resident;
      P.cfg = c;
      found = true;
    }
  }
  if (!found) {
    if (P.mode == relattn::kRelT5 || P.mode == relattn::kRelGrid)
      return fail(RELATTN_ERR_UNSUPPORTED,
                  "scalar-bias offset window 2*min(max_distance or window, n-1)+1 = %d "
                  "does not fit on chip",
                  2 * p.t5_dist + 1);
    if (P.mode == relattn::kRelGraph)
      return fail(RELATTN_ERR_UNSUPPORTED, "rows of %d labels per query do not fit on chip",
                  p.nr);
    return fail(RELATTN_ERR_UNSUPPORTED,
                "label window of %d rows (2*clip_k+1 clipped to 2n-1) does not fit on chip",
                p.nr);
  }
  const int br = 32 * P.cfg.waves;
  p.n_qtiles = (int32_t)((n + br - 1) / br);
  p.nstage = P.cfg.nstage;
  p.wv_mode = P.cfg.wv_mode;
  {
    // stage loads address a tile's rows by 32-bit byte offsets from its first
    // row when that range fits
    const int64_t esz = P.bf16 ? 2 : 4;
    const int64_t span_k = (int64_t)P.cfg.kblock * k->stride[2] * esz;
    const int64_t span_v = (int64_t)P.cfg.kblock * v->stride[2] * esz;
    p.dma32 = (span_k < (int64_t)1 << 31 && span_v < (int64_t)1 << 31) ? 1 : 0;
  }
  if (B * H * (int64_t)p.n_qtiles > INT32_MAX)
    return fail(RELATTN_ERR_UNSUPPORTED, "too many workgroups (B*H*ceil(n/%d))", br);
  {
    // x / d as (umulhi(x, m) + x) >> s for every x < 2^31: s = ceil(log2 d),
    // m = floor(2^32 (2^s - d) / d) + 1
    auto divisor = [](int64_t d, uint32_t* m, int32_t* sh) {
      if (d < 1) d = 1;
      int e = 0;
      while ((int64_t(1) << e) < d) ++e;
      *m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << e) - (uint64_t)d)) / (uint64_t)d + 1);
      *sh = e;
    };
    const int64_t grid = B * H * p.n_qtiles;
    const int64_t hpx = (grid % 8 == 0) ? (grid / 8) / p.n_qtiles : 1;
    divisor(H, &p.dv_h_m, &p.dv_h_s);
    divisor(p.n_qtiles, &p.dv_qt_m, &p.dv_qt_s);
    divisor(hpx, &p.dv_hpx_m, &p.dv_hpx_s);
  }

  p.q = q->data;
  p.k = k->data;
  p.v = v->data;
  p.o = out->data;
  p.q_sb = q->stride[0]; p.q_sh = q->stride[1]; p.q_sn = q->stride[2];
  p.k_sb = k->stride[0]; p.k_sh = k->stride[1]; p.k_sn = k->stride[2];
  p.v_sb = v->stride[0]; p.v_sh = v->stride[1]; p.v_sn = v->stride[2];
  p.o_sb = out->stride[0]; p.o_sh = out->stride[1]; p.o_sn = out->stride[2];
  if (wK) {
    p.wk = wK->data;
    p.wk_sh = wK->shape[0] == 1 ? 0 : wK->stride[0];
    p.wk_sr = wK->stride[1];
  }
  if (is_xl && P.mode == relattn::kRelXL) {
    // fused: the kernel reads R's row of distance i - j (clamped to +-clip)
    // from the row of distance 0
    const int64_t esz = P.bf16 ? 2 : 4;
    p.wk = static_cast<const char*>(wK->data) + (int64_t)clip_k * wK->stride[1] * esz;
    p.wk_sr = wK->stride[1];
    p.xl = 1;
    p.xl_u = xl_u->data;
    p.xl_v = xl_v->data;
    p.xl_u_sh = xl_u->shape[0] == 1 ? 0 : xl_u->stride[0];
    p.xl_v_sh = xl_v->shape[0] == 1 ? 0 : xl_v->stride[0];
  } else if (is_xl) {
    // row r of the label window (offset j - i = r - clip) is R's row for
    // distance i - j, 2*clip - r: start at the last row and step backwards
    const int64_t esz = P.bf16 ? 2 : 4;
    p.wk = static_cast<const char*>(wK->data) + 2 * (int64_t)clip_k * wK->stride[1] * esz;
    p.wk_sr = -wK->stride[1];
    p.xl = 1;
    p.xl_u = xl_u->data;
    p.xl_v = xl_v->data;
    p.xl_u_sh = xl_u->shape[0] == 1 ? 0 : xl_u->stride[0];
    p.xl_v_sh = xl_v->shape[0] == 1 ? 0 : xl_v->stride[0];
  }
  if (wV) {
    p.wv = wV->data;
    p.wv_sh = wV->shape[0] == 1 ? 0 : wV->stride[0];
    p.wv_sr = wV->stride[1];
  }
  if (is_t5) {
    p.t5_bias = static_cast<const float*>(t5_bias->data);
    p.tb_sb = t5_bias->stride[0];
    p.tb_sh = t5_bias->stride[1];
  }
  if (is_ob) {
    p.t5_bias = static_cast<const float*>(ob->data);
    p.tb_sb = ob->stride[1];
    p.tb_sh = ob->shape[0] == 1 ? 0 : ob->stride[0];
  }
  return RELATTN_OK;
}

// ---- incremental decoding --------------------------------------------------

struct DecPlan {
  bool empty = false;
  bool bf16 = false;
  int d = 0;
  RelMode mode = relattn::kRelNone;
  bool has_wk = false, has_wv = false;
  size_t ws_bytes = 0;
  size_t ws_o_off = 0, ws_band_off = 0;  // byte offsets in the workspace
  relattn::DecParams p{};
};

size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

int make_dec_plan(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                  const relattn_tensor* wK, const relattn_tensor* wV,
                  const relattn_tensor* t5_bias, const relattn_t5_params* t5, int32_t clip_k,
                  float scale, const relattn_tensor* out, DecPlan* plan, bool want_t5_table,
                  const relattn_tensor* ob = nullptr, int32_t ob_window = 0,
                  const relattn_tensor* xl_u = nullptr, const relattn_tensor* xl_v = nullptr) {
  int st;
  if ((st = check_view(q, "q", 4, true))) return st;
  if ((st = check_view(k, "k", 4, true))) return st;
  if ((st = check_view(v, "v", 4, true))) return st;
  if ((st = check_view(out, "out", 4, true))) return st;
  const relattn_tensor* others[3] = {k, v, out};
  const char* names[3] = {"k", "v", "out"};
  for (int t = 0; t < 3; ++t)
    if (others[t]->dtype != q->dtype)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s dtype differs from q", names[t]);
  for (int i = 0; i < 4; ++i)
    if (out->shape[i] != q->shape[i])
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "out shape differs from q in dim %d", i);
  for (int t = 0; t < 2; ++t)
    for (int i : {0, 1, 3})
      if (others[t]->shape[i] != q->shape[i])
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s shape differs from q in dim %d",
                    names[t], i);
  if (v->shape[2] != k->shape[2])
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "k and v caches differ in length");
  const int64_t B = q->shape[0], H = q->shape[1], Tq = q->shape[2], d = q->shape[3];
  const int64_t L = k->shape[2];
  if (!(d == 16 || d == 32 || d == 64 || d == 128))
    return fail(RELATTN_ERR_UNSUPPORTED, "head size d = %lld is not one of 16, 32, 64, 128",
                (long long)d);
  if (L > kMaxSeq || Tq > kMaxSeq)
    return fail(RELATTN_ERR_UNSUPPORTED, "cache or query length exceeds 2^30");
  if (std::isnan(scale) || std::isinf(scale))
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "scale must be finite");
  const bool is_t5 = t5_bias != nullptr || t5 != nullptr;
  if ((t5_bias == nullptr) != (t5 == nullptr))
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "t5_bias and t5 params must be given together");
  if (is_t5 && (wK || wV))
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "T5 bias excludes the wK/wV tables");
  if (!is_t5 && clip_k < 0) return fail(RELATTN_ERR_INVALID_ARGUMENT, "clip_k must be >= 0");
  if (!is_t5 && (int64_t)clip_k > kMaxSeq)
    return fail(RELATTN_ERR_UNSUPPORTED, "clip_k exceeds 2^30");
  const bool is_xl = xl_u != nullptr || xl_v != nullptr;
  if (is_xl) {
    // Transformer-XL: wK is the position table R (by distance i - j), u and v
    // the global biases; no value table, no scalar bias
    if (!xl_u || !xl_v || !wK)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "R, u and v must be given together");
    if (wV || is_t5 || ob)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "Transformer-XL logits exclude the other tables");
    const relattn_tensor* uv[2] = {xl_u, xl_v};
    const char* nm[2] = {"u", "v"};
    for (int t = 0; t < 2; ++t) {
      if ((st = check_view(uv[t], nm[t], 2, true))) return st;
      if (uv[t]->dtype != q->dtype)
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s dtype differs from q", nm[t]);
      if (!(uv[t]->shape[0] == H || uv[t]->shape[0] == 1) || uv[t]->shape[1] != d)
        return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s must be [H or 1, d]", nm[t]);
    }
  }
  if (wK && (st = check_table(wK, is_xl ? "R" : "wK", q, clip_k))) return st;
  if (wV && (st = check_table(wV, "wV", q, clip_k))) return st;
  T5Buckets tb = {};
  if (is_t5) {
    if ((st = check_view(t5_bias, "t5_bias", 2, false))) return st;
    if (t5_bias->dtype != RELATTN_F32)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "t5_bias must be F32");
    if (t5_bias->shape[0] != t5->num_buckets || t5_bias->shape[1] != H)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "t5_bias must be [num_buckets, H]");
    if ((st = check_t5(t5, want_t5_table ? &tb : nullptr))) return st;
  }

  DecPlan& P = *plan;
  P.bf16 = q->dtype == RELATTN_BF16;
  P.d = (int)d;
  const bool is_ob = ob != nullptr;  // scalar bias by clipped offset
  if (is_ob) {
    if (wK || wV || is_t5)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "an offset bias excludes the other tables");
    if ((st = check_view(ob, "bias", 2, false))) return st;
    if (ob->dtype != RELATTN_F32) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias must be F32");
    if (ob_window < 0) return fail(RELATTN_ERR_INVALID_ARGUMENT, "window must be >= 0");
    if ((int64_t)ob_window > kMaxSeq) return fail(RELATTN_ERR_UNSUPPORTED, "window exceeds 2^30");
    if (!(ob->shape[0] == q->shape[1] || ob->shape[0] == 1))
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias: shape[0] must be H (%lld) or 1",
                  (long long)q->shape[1]);
    if (ob->shape[1] != 2 * (int64_t)ob_window + 1)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias: shape[1] must be 2*window+1 = %lld",
                  (long long)(2 * (int64_t)ob_window + 1));
  }
  P.mode = is_xl ? relattn::kRelXL
                 : (is_t5 || is_ob) ? relattn::kRelT5
                                    : ((wK || wV) ? relattn::kRelShaw : relattn::kRelNone);
  P.has_wk = wK != nullptr;
  P.has_wv = wV != nullptr;
  P.empty = (B == 0 || H == 0 || Tq == 0);
  if (P.empty) return RELATTN_OK;
  const int64_t rows = B * H * Tq;
  if (rows > INT32_MAX) return fail(RELATTN_ERR_UNSUPPORTED, "too many query rows (B*H*Tq)");
  const int ch = relattn::dec_chunk(P.bf16 ? 2 : 4, P.d);
  const int64_t nch = std::max<int64_t>(1, (L + ch - 1) / ch);
  if (nch > 65535)
    return fail(RELATTN_ERR_UNSUPPORTED, "cache of %lld rows exceeds %lld", (long long)L,
                (long long)65535 * ch);
  const int64_t nband = (P.mode == relattn::kRelShaw && P.has_wv)
                            ? std::min<int64_t>(clip_k, std::max<int64_t>(L, 1))
                            : 0;
  // Split each row's cache over just enough workgroups to give the launch
  // about kDecTargetWgs of them; a row held by one workgroup needs no
  // partial results (and no workspace) when its single-key labels fit in LDS.
  int64_t nsp = std::min<int64_t>(nch, (relattn::kDecTargetWgs + rows - 1) / rows);
  const int64_t cps = (nch + nsp - 1) / nsp;
  nsp = (nch + cps - 1) / cps;
  const bool direct = nsp == 1 && nband <= relattn::kDirectBand;
  if (!direct) {
    P.ws_o_off = align16((size_t)rows * nsp * 2 * sizeof(float));
    P.ws_band_off = P.ws_o_off + (size_t)rows * nsp * d * sizeof(float);
    P.ws_bytes = align16(P.ws_band_off + (size_t)rows * nband * sizeof(float));
  }

  relattn::DecParams& p = P.p;
  p.B = (int32_t)B;
  p.H = (int32_t)H;
  p.Tq = (int32_t)Tq;
  p.L = (int32_t)L;
  p.clip = (is_t5 || is_ob) ? 0 : clip_k;
  p.nband = (int32_t)nband;
  p.nch = (int32_t)nch;
  p.cps = (int32_t)cps;
  p.nsp = (int32_t)nsp;
  p.direct = direct ? 1 : 0;
  p.t5 = tb;
  const float s = scale > 0.f ? scale : (is_t5 ? 1.f : 1.f / std::sqrt((float)d));
  p.scale_log2 = s * 1.4426950408889634f;
  if (is_xl) {
    p.xl_u = xl_u->data;
    p.xl_v = xl_v->data;
    p.xl_u_sh = xl_u->shape[0] == 1 ? 0 : xl_u->stride[0];
    p.xl_v_sh = xl_v->shape[0] == 1 ? 0 : xl_v->stride[0];
  }
  if (is_ob) {
    // the bias of offset delta is entry clip(delta, W) + W of the head's row
    p.ob = 1;
    p.ob_w = ob_window;
    p.t5_bias = static_cast<const float*>(ob->data);
    p.tb_sb = ob->stride[1];
    p.tb_sh = ob->shape[0] == 1 ? 0 : ob->stride[0];
  }
  p.q = q->data;
  p.k = k->data;
  p.v = v->data;
  p.o = out->data;
  p.q_sb = q->stride[0]; p.q_sh = q->stride[1]; p.q_st = q->stride[2];
  p.k_sb = k->stride[0]; p.k_sh = k->stride[1]; p.k_sn = k->stride[2];
  p.v_sb = v->stride[0]; p.v_sh = v->stride[1]; p.v_sn = v->stride[2];
  p.o_sb = out->stride[0]; p.o_sh = out->stride[1]; p.o_st = out->stride[2];
  if (wK) {
    p.wk = wK->data;
    p.wk_sh = wK->shape[0] == 1 ? 0 : wK->stride[0];
    p.wk_sr = wK->stride[1];
  }
  if (wV) {
    p.wv = wV->data;
    p.wv_sh = wV->shape[0] == 1 ? 0 : wV->stride[0];
    p.wv_sr = wV->stride[1];
  }
  if (is_t5) {
    p.t5_bias = static_cast<const float*>(t5_bias->data);
    p.tb_sb = t5_bias->stride[0];
    p.tb_sh = t5_bias->stride[1];
  }
  return RELATTN_OK;
}

// The device the calling thread has selected must be a gfx950.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(RELATTN_ERR_NO_DEVICE, "no HIP device available");
  }
  static std::atomic<int> known[64];  // 0 unknown, 1 gfx950, 2 other
  const int slot = dev < 64 ? dev : -1;
  int state = slot >= 0 ? known[slot].load(std::memory_order_relaxed) : 0;
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(RELATTN_ERR_NO_DEVICE, "cannot query HIP device %d", dev);
    }
    state = std::string(prop.gcnArchName).rfind("gfx950", 0) == 0 ? 1 : 2;
    if (slot >= 0) known[slot].store(state, std::memory_order_relaxed);
  }
  if (state != 1) return fail(RELATTN_ERR_UNSUPPORTED, "device %d is not a gfx950", dev);
  return RELATTN_OK;
}

// ---- backward ---------------------------------------------------------------

int check_like_q(const relattn_tensor* t, const char* name, const relattn_tensor* q) {
  int st = check_view(t, name, 4, true);
  if (st) return st;
  if (t->dtype != q->dtype) return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s dtype differs from q", name);
  for (int i = 0; i < 4; ++i)
    if (t->shape[i] != q->shape[i])
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s shape differs from q in dim %d", name, i);
  return RELATTN_OK;
}

int check_f32(const relattn_tensor* t, const char* name, int ndim, const int64_t* shape) {
  int st = check_view(t, name, ndim, false);
  if (st) return st;
  if (t->dtype != RELATTN_F32) return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s must be F32", name);
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] != shape[i])
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "%s: shape[%d] must be %lld, got %lld", name, i,
                  (long long)shape[i], (long long)t->shape[i]);
  return RELATTN_OK;
}

// lse output/input of shape [B, H, n]
int check_lse(const relattn_tensor* lse, const relattn_tensor* q) {
  if (!lse) return fail(RELATTN_ERR_INVALID_ARGUMENT, "lse is NULL");
  const int64_t shp[3] = {q->shape[0], q->shape[1], q->shape[2]};
  return check_f32(lse, "lse", 3, shp);
}

struct BwdPlan {
  Plan fwd;
  relattn::BwdCfg cfg{};
  relattn::BwdParams p{};
  size_t ws_bytes = 0;
  size_t off_stat = 0, off_pk = 0, off_pv = 0, off_pb = 0, off_pu = 0;
};

int make_bwd_plan(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                  const relattn_tensor* wK, const relattn_tensor* wV,
                  const relattn_tensor* t5_bias, const relattn_t5_params* t5, int32_t clip_k,
                  float scale, const relattn_mask* mask, const relattn_tensor* out,
                  const relattn_tensor* dout, const relattn_tensor* lse,
                  const relattn_tensor* dq, const relattn_tensor* dk, const relattn_tensor* dv,
                  const relattn_tensor* dwK, const relattn_tensor* dwV,
                  const relattn_tensor* dbias, BwdPlan* plan, bool want_t5_table,
                  const relattn_tensor* ob = nullptr, int32_t ob_window = 0,
                  int32_t grid_m = 0, const relattn_tensor* labels = nullptr,
                  const relattn_tensor* xl_u = nullptr, const relattn_tensor* xl_v = nullptr,
                  const relattn_tensor* du = nullptr, const relattn_tensor* dvb = nullptr) {
  Plan& F = plan->fwd;
  int st = make_plan(q, k, v, wK, wV, t5_bias, t5, clip_k, scale, mask, out, &F, want_t5_table,
                     ob, ob_window, xl_u, xl_v, grid_m, labels);
  if (st) return st;
  // Transformer-XL: the backward runs the key-table path with R as the table
  const bool xl = xl_u != nullptr;
  if (xl) {
    F.mode = relattn::kRelXL;
    F.has_wk = true;
    F.has_wv = false;
  }
  {
    const int64_t d0 = q->shape[3];
    if ((du || dvb) && !xl)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "du / dv given without Transformer-XL biases");
    if (du) {
      const int64_t shp[2] = {xl_u->shape[0], d0};
      if ((st = check_f32(du, "du", 2, shp))) return st;
      if (numel(du) > 0 && du->stride[1] != 1)
        return fail(RELATTN_ERR_UNSUPPORTED, "du: innermost dimension must be contiguous");
    }
    if (dvb) {
      const int64_t shp[2] = {xl_v->shape[0], d0};
      if ((st = check_f32(dvb, "dv", 2, shp))) return st;
      if (numel(dvb) > 0 && dvb->stride[1] != 1)
        return fail(RELATTN_ERR_UNSUPPORTED, "dv: innermost dimension must be contiguous");
    }
  }
  if ((st = check_like_q(dout, "dout", q))) return st;
  if ((st = check_like_q(dq, "dq", q))) return st;
  if ((st = check_like_q(dk, "dk", q))) return st;
  if ((st = check_like_q(dv, "dv", q))) return st;
  if ((st = check_lse(lse, q))) return st;
  const int64_t B = q->shape[0], H = q->shape[1], n = q->shape[2], d = q->shape[3];
  // table rows: 2 clip + 1 labels by clipped offset, NL by edge label
  const bool graph = F.mode == relattn::kRelGraph;
  if (dwK) {
    if (!wK) return fail(RELATTN_ERR_INVALID_ARGUMENT, "dwK given without wK");
    const int64_t shp[3] = {wK->shape[0], graph ? wK->shape[1] : 2 * (int64_t)clip_k + 1, d};
    if ((st = check_f32(dwK, "dwK", 3, shp))) return st;
  }
  if (dwV) {
    if (!wV) return fail(RELATTN_ERR_INVALID_ARGUMENT, "dwV given without wV");
    const int64_t shp[3] = {wV->shape[0], graph ? wV->shape[1] : 2 * (int64_t)clip_k + 1, d};
    if ((st = check_f32(dwV, "dwV", 3, shp))) return st;
  }
  if (dbias) {
    if (!t5_bias && !ob)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "dbias given without a bias table");
    const int64_t shp[2] = {t5_bias ? t5_bias->shape[0] : ob->shape[0],
                            t5_bias ? t5_bias->shape[1] : ob->shape[1]};
    if ((st = check_f32(dbias, "dbias", 2, shp))) return st;
  }
  if (F.empty) return RELATTN_OK;

  const relattn::FwdParams& f = F.p;
  relattn::BwdParams& p = plan->p;
  relattn::BwdCfg& cfg = plan->cfg;
  cfg = relattn::bwd_cfg(F.bf16, F.d, false, false);
  p.B = f.B;
  p.H = f.H;
  p.n = f.n;
  p.d = (int32_t)d;
  p.n_pad = (int32_t)((n + 63) / 64 * 64);
  p.clip = f.clip;
  p.r_lo = f.r_lo;
  p.nr = f.nr;
  p.htk = wK ? (int32_t)wK->shape[0] : 0;
  p.htv = wV ? (int32_t)wV->shape[0] : 0;
  p.hb = ob ? (int32_t)ob->shape[0] : (int32_t)H;
  p.causal = f.causal;
  p.key_lens = f.key_lens;
  const bool is_t5 = t5_bias != nullptr;
  p.scale = scale > 0.f ? scale : (is_t5 ? 1.f : 1.f / std::sqrt((float)d));
  p.scale_log2 = f.scale_log2;
  p.t5_dist = f.t5_dist;
  p.ob = f.ob;
  p.ob_lo = f.ob_lo;
  p.ob_n = ob ? 2 * ob_window + 1 : 0;
  const bool grid = F.mode == relattn::kRelGrid, lab = F.mode == relattn::kRelLabel;
  if (grid) {
    // the table's (2M - 1)^2 entries, summed like an offset table of that many
    p.ob_n = f.t5.nb;
    p.grid_m = f.grid_m;
    p.grid_inv = f.grid_inv;
  }
  if (lab) {
    // the table's NL entries, one per label
    p.ob_n = f.t5.nb;
    p.lab = f.lab;
    p.lab_sb = f.lab_sb;
    p.lab_sn = f.lab_sn;
  }
  if (graph) {
    // the tables' NL rows, one per label
    p.nlab = f.nr;
    p.lab = f.lab;
    p.lab_sb = f.lab_sb;
    p.lab_sn = f.lab_sn;
  }
  p.t5 = f.t5;
  p.t5_bias = f.t5_bias;
  p.tb_sb = f.tb_sb;
  p.tb_sh = f.tb_sh;
  p.q = f.q;
  p.k = f.k;
  p.v = f.v;
  p.o = f.o;
  p.wk = f.wk;
  p.wv = f.wv;
  p.wk_sh = f.wk_sh;
  p.wk_sr = f.wk_sr;
  p.wv_sh = f.wv_sh;
  p.wv_sr = f.wv_sr;
  p.q_sb = f.q_sb; p.q_sh = f.q_sh; p.q_sn = f.q_sn;
  p.k_sb = f.k_sb; p.k_sh = f.k_sh; p.k_sn = f.k_sn;
  p.v_sb = f.v_sb; p.v_sh = f.v_sh; p.v_sn = f.v_sn;
  p.o_sb = f.o_sb; p.o_sh = f.o_sh; p.o_sn = f.o_sn;
  p.dout = dout->data;
  p.do_sb = dout->stride[0]; p.do_sh = dout->stride[1]; p.do_sn = dout->stride[2];
  p.dq = dq->data;
  p.dq_sb = dq->stride[0]; p.dq_sh = dq->stride[1]; p.dq_sn = dq->stride[2];
  p.dk = dk->data;
  p.dk_sb = dk->stride[0]; p.dk_sh = dk->stride[1]; p.dk_sn = dk->stride[2];
  p.dv = dv->data;
  p.dv_sb = dv->stride[0]; p.dv_sh = dv->stride[1]; p.dv_sn = dv->stride[2];
  p.lse = static_cast<const float*>(lse->data);
  p.lse_sb = lse->stride[0];
  p.lse_sh = lse->stride[1];
  if ((lse->stride[2]) != 1)
    return fail(RELATTN_ERR_UNSUPPORTED, "lse: innermost dimension must be contiguous");
  if (dwK) {
    p.dwk = static_cast<float*>(dwK->data);
    p.dwk_sh = dwK->stride[0];
    p.dwk_sr = dwK->stride[1];
  }
  if (dwV) {
    p.dwv = static_cast<float*>(dwV->data);
    p.dwv_sh = dwV->stride[0];
    p.dwv_sr = dwV->stride[1];
  }
  if (dbias) {
    p.db = static_cast<float*>(dbias->data);
    p.db_s0 = dbias->stride[0];
    p.db_s1 = dbias->stride[1];
  }
  if (xl) {
    // the table row of label r (offset j - i = r - c) is R's row of distance
    // i - j, 2c - r: start at R's last row and step backwards (the gradient
    // table the same way)
    const int64_t c = clip_k;
    const int64_t r_lo = std::max<int64_t>(0, c - (n - 1));
    const int64_t r_hi = f.causal ? c : std::min<int64_t>(2 * c, c + n - 1);
    p.clip = (int32_t)c;
    p.r_lo = (int32_t)r_lo;
    p.nr = (int32_t)(r_hi - r_lo + 1);
    const int64_t esz = F.bf16 ? 2 : 4;
    p.wk = static_cast<const char*>(wK->data) + 2 * c * wK->stride[1] * esz;
    p.wk_sr = -wK->stride[1];
    p.wk_sh = wK->shape[0] == 1 ? 0 : wK->stride[0];
    p.htk = (int32_t)wK->shape[0];
    p.xl_u = xl_u->data;
    p.xl_v = xl_v->data;
    p.xl_u_sh = xl_u->shape[0] == 1 ? 0 : xl_u->stride[0];
    p.xl_v_sh = xl_v->shape[0] == 1 ? 0 : xl_v->stride[0];
    if (dwK) {
      p.dwk = static_cast<float*>(dwK->data) + 2 * c * dwK->stride[1];
      p.dwk_sr = -dwK->stride[1];
    }
    if (du) {
      p.du = static_cast<float*>(du->data);
      p.du_sh = du->stride[0];
      p.hu = (int32_t)xl_u->shape[0];
    }
    if (dvb) {
      p.dvb = static_cast<float*>(dvb->data);
      p.dvb_sh = dvb->stride[0];
      p.hv = (int32_t)xl_v->shape[0];
    }
  }
  const bool shaw = F.mode == relattn::kRelShaw || xl || graph, t5m = F.mode == relattn::kRelT5;
  const bool want_db = (t5m || grid || lab) && dbias != nullptr;
  // the wide workgroup shapes unless their LDS does not fit
  size_t lq = relattn::bwd_lds_q(F.bf16, F.d, cfg, F.mode, F.has_wk, F.has_wv, p.nr, p.t5_dist,
                                 p.t5.nb, want_db);
  size_t lkv = relattn::bwd_lds_kv(F.bf16, F.d, cfg, F.mode, F.has_wk, F.has_wv, p.nr,
                                   p.t5_dist, p.t5.nb);
  if (lq > kMaxLdsBytes || lkv > kMaxLdsBytes) {
    cfg = relattn::bwd_cfg(F.bf16, F.d, lq > kMaxLdsBytes, lkv > kMaxLdsBytes);
    lq = relattn::bwd_lds_q(F.bf16, F.d, cfg, F.mode, F.has_wk, F.has_wv, p.nr, p.t5_dist,
                            p.t5.nb, want_db);
    lkv = relattn::bwd_lds_kv(F.bf16, F.d, cfg, F.mode, F.has_wk, F.has_wv, p.nr, p.t5_dist,
                              p.t5.nb);
    // the key table alone in bf16 at d <= 64: one wave and 32-key tiles
    if (lq > kMaxLdsBytes && F.bf16 && F.d <= 64 && shaw && F.has_wk && !F.has_wv) {
      cfg = relattn::bwd_cfg(F.bf16, F.d, true, lkv > kMaxLdsBytes || cfg.kqblock != 64, true);
      lq = relattn::bwd_lds_q(F.bf16, F.d, cfg, F.mode, F.has_wk, F.has_wv, p.nr, p.t5_dist,
                              p.t5.nb, want_db);
    }
  }
  // short sequences: no dq workgroup wider than the rows there are
  if (n <= 64 && cfg.qwaves == 4 && lq <= kMaxLdsBytes) {
    const relattn::BwdCfg narrow = relattn::bwd_cfg(F.bf16, F.d, true, cfg.kqblock == 32);
    const size_t ln = relattn::bwd_lds_q(F.bf16, F.d, narrow, F.mode, F.has_wk, F.has_wv, p.nr,
                                         p.t5_dist, p.t5.nb, want_db);
    if (narrow.qwaves == 2 && ln <= kMaxLdsBytes) {
      cfg.qwaves = narrow.qwaves;
      cfg.qkblock = narrow.qkblock;
      lq = ln;
    }
  }
  const int64_t brq = 32 * cfg.qwaves, brk = 32 * cfg.kwaves;
  p.n_qtiles = (int32_t)((n + brq - 1) / brq);
  p.n_ktiles = (int32_t)((n + brk - 1) / brk);
  if (B * H * (int64_t)std::max(p.n_qtiles, p.n_ktiles) > INT32_MAX)
    return fail(RELATTN_ERR_UNSUPPORTED, "too many workgroups");
  if (lq > kMaxLdsBytes || lkv > kMaxLdsBytes)
    return fail(RELATTN_ERR_UNSUPPORTED,
                "backward: per-workgroup state of %zu / %zu bytes exceeds on-chip memory "
                "(label window %d rows, offset window %d)",
                lq, lkv, p.nr, 2 * p.t5_dist + 1);

  // workspace sections (fp32), 256-byte aligned
  size_t off = 0;
  auto take = [&](int64_t floats) {
    const size_t at = off;
    off += ((size_t)floats * 4 + 255) / 256 * 256;
    return at;
  };
  const int64_t BH = B * H;
  plan->off_stat = take(BH * 2 * p.n_pad + 64);
  plan->off_pk = (shaw && F.has_wk) ? take(BH * p.n_qtiles * p.nr * d) : 0;
  plan->off_pv = (shaw && F.has_wv) ? take(BH * p.n_qtiles * p.nr * d) : 0;
  plan->off_pb = want_db ? take(BH * p.n_qtiles * p.t5.nb) : 0;
  plan->off_pu = (xl && (du || dvb)) ? take(BH * p.n_qtiles * 2 * d) : 0;
  plan->ws_bytes = off;
  return RELATTN_OK;
}

int run_bwd(BwdPlan& plan, const relattn_tensor* wK, const relattn_tensor* wV, bool want_db,
            void* workspace, size_t workspace_bytes, void* stream) {
  if (plan.fwd.empty) return RELATTN_OK;
  if (workspace_bytes < plan.ws_bytes)
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "workspace of %zu bytes, %zu needed",
                workspace_bytes, plan.ws_bytes);
  if (!workspace || !aligned16(workspace))
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "workspace is NULL or not 16-byte aligned");
  int st;
  if ((st = check_device())) return st;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  relattn::BwdParams& p = plan.p;
  const bool xl = plan.fwd.mode == relattn::kRelXL;
  const bool shaw = plan.fwd.mode == relattn::kRelShaw || xl ||
                    plan.fwd.mode == relattn::kRelGraph;
  p.ws_stat = reinterpret_cast<float*>(ws + plan.off_stat);
  p.ws_pk = (shaw && wK) ? reinterpret_cast<float*>(ws + plan.off_pk) : nullptr;
  p.ws_pu = (xl && (p.du || p.dvb)) ? reinterpret_cast<float*>(ws + plan.off_pu) : nullptr;
  p.ws_pv = (shaw && wV) ? reinterpret_cast<float*>(ws + plan.off_pv) : nullptr;
  p.ws_pb = want_db ? reinterpret_cast<float*>(ws + plan.off_pb) : nullptr;
  const int e = relattn::launch_bwd(plan.fwd.bf16, plan.fwd.d, plan.cfg, plan.fwd.mode,
                                    plan.fwd.has_wk, plan.fwd.has_wv, p, stream);
  if (e != (int)hipSuccess)
    return fail(RELATTN_ERR_LAUNCH_FAILED, "launch failed: %s", hipGetErrorString((hipError_t)e));
  return RELATTN_OK;
}

// Enqueue the forward launch of a made plan (nothing for an empty problem).
int run_fwd(const Plan& plan, void* stream) {
  int st;
  if ((st = check_device())) return st;
  if (plan.empty) return RELATTN_OK;
  const int e = plan.cfg.lean == 3
                    ? relattn::launch_window_grid(plan.d, plan.p, stream)
                : plan.cfg.lean
                    ? relattn::launch_fwd_lean(plan.d, plan.cfg, plan.mode, plan.has_wk,
                                               plan.has_wv, plan.p, stream)
                    : relattn::launch_fwd(plan.bf16, plan.d, plan.cfg, plan.mode, plan.has_wk,
                                          plan.has_wv, plan.p, stream);
  if (e != (int)hipSuccess)
    return fail(RELATTN_ERR_LAUNCH_FAILED, "launch failed: %s", hipGetErrorString((hipError_t)e));
  return RELATTN_OK;
}

// Check the cache lengths and workspace of a made decode plan, then enqueue it.
// ---- scratch of the entry points that allocate nothing ----------------------
// One file-scope array per device (each GPU the library runs on holds its own
// copy until the process ends).  Host code never uses the array's name as an
// address: hipGetSymbolAddress resolves this device's copy once, with that
// device current, and the pointer is kept per device.
constexpr size_t kScratchBytes = size_t(4) << 20;
}  // namespace
namespace relattn {
__device__ __align__(256) unsigned char scratch[kScratchBytes];
}  // namespace relattn
namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxScratchDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(RELATTN_ERR_NO_DEVICE, "no HIP device available");
  }
  if (dev >= kMaxScratchDevices)
    return fail(RELATTN_ERR_UNSUPPORTED, "device ordinal %d exceeds %d", dev,
                kMaxScratchDevices - 1);
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* a = nullptr;
      const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(relattn::scratch));
      if (e != hipSuccess || !a) {
        (void)hipGetLastError();
        return fail(RELATTN_ERR_LAUNCH_FAILED, "cannot resolve the scratch array on device %d: %s",
                    dev, hipGetErrorString(e));
      }
      g_scratch_addr[dev].store(a, std::memory_order_release);
      p = a;
    }
  }
  *out = p;
  return RELATTN_OK;
}

int run_decode(DecPlan& plan, const int32_t* cache_lens, void* workspace,
               size_t workspace_bytes, void* stream) {
  if (cache_lens && (reinterpret_cast<uintptr_t>(cache_lens) & 3u))
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "cache_lens is not 4-byte aligned");
  if (!plan.empty && plan.ws_bytes > 0) {
    if (workspace_bytes < plan.ws_bytes)
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "workspace of %zu bytes, %zu needed",
                  workspace_bytes, plan.ws_bytes);
    if (!workspace || !aligned16(workspace))
      return fail(RELATTN_ERR_INVALID_ARGUMENT, "workspace is NULL or not 16-byte aligned");
  }
  int st;
  if ((st = check_device())) return st;
  if (plan.empty) return RELATTN_OK;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  plan.p.cache_lens = cache_lens;
  plan.p.ws_ml = reinterpret_cast<float*>(ws);
  plan.p.ws_o = reinterpret_cast<float*>(ws + plan.ws_o_off);
  plan.p.ws_band = reinterpret_cast<float*>(ws + plan.ws_band_off);
  const int e = relattn::launch_decode(plan.bf16, plan.d, plan.mode, plan.has_wk, plan.has_wv,
                                       plan.p, stream);
  if (e != (int)hipSuccess)
    return fail(RELATTN_ERR_LAUNCH_FAILED, "launch failed: %s",
                hipGetErrorString((hipError_t)e));
  return RELATTN_OK;
}

int run_fwd_lse(Plan& plan, const relattn_tensor* lse, void* stream) {
  if (plan.empty) return RELATTN_OK;
  if (lse->stride[2] != 1)
    return fail(RELATTN_ERR_UNSUPPORTED, "lse: innermost dimension must be contiguous");
  plan.p.lse = static_cast<float*>(lse->data);
  plan.p.lse_sb = lse->stride[0];
  plan.p.lse_sh = lse->stride[1];
  return run_fwd(plan, stream);
}

// ---- plan cache of the forward -------------------------------------------
// A forward plan depends on the arguments' dtypes, shapes, strides and scalars,
// and on the data pointers only through their nullness and 16-byte alignment.
// Each thread keeps its last few plans keyed on exactly those facts: a hit
// copies the cached plan and substitutes the call's pointers, so a repeated
// call costs a key comparison instead of the validation and the search over
// launch shapes.  The cache is thread-local (no locks) and a fixed array (no
// allocation); only plans that passed every check are stored.
struct TensorKey {
  int64_t shape[4], stride[4];
  int32_t dtype, ndim;
  uint32_t ptr_bits;  // 0: NULL view; else 1 + (data & 15), or 32 for a non-NULL view without data
};
struct FwdKey {
  TensorKey t[7];  // q, k, v, wK, wV, t5_bias, out
  relattn_t5_params t5;
  int32_t has_t5, clip, causal, has_mask;
  uint32_t lens_bits;  // 0: no key lengths; else 1 + (pointer & 3)
  float scale;
};

bool make_tensor_key(const relattn_tensor* t, TensorKey* k) {
  if (!t) return true;  // stays all zero
  if (t->ndim < 0 || t->ndim > 4) return false;
  k->dtype = t->dtype;
  k->ndim = t->ndim;
  for (int i = 0; i < t->ndim; ++i) {
    k->shape[i] = t->shape[i];
    k->stride[i] = t->stride[i];
  }
  const uintptr_t a = reinterpret_cast<uintptr_t>(t->data);
  k->ptr_bits = a ? 1u + (uint32_t)(a & 15u) : 32u;
  return true;
}

bool make_fwd_key(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                  const relattn_tensor* wK, const relattn_tensor* wV,
                  const relattn_tensor* t5_bias, const relattn_t5_params* t5, int32_t clip_k,
                  float scale, const relattn_mask* mask, const relattn_tensor* out,
                  FwdKey* key) {
  // cleared whole, padding included, so that keys compare with memcmp
  std::memset(key, 0, sizeof *key);
  const relattn_tensor* ts[7] = {q, k, v, wK, wV, t5_bias, out};
  for (int i = 0; i < 7; ++i)
    if (!make_tensor_key(ts[i], &key->t[i])) return false;
  if (t5) {
    key->t5 = *t5;
    key->has_t5 = 1;
  }
  key->clip = clip_k;
  key->scale = scale;
  if (mask) {
    key->has_mask = 1;
    key->causal = mask->causal;
    const uintptr_t a = reinterpret_cast<uintptr_t>(mask->key_lens);
    key->lens_bits = a ? 1u + (uint32_t)(a & 3u) : 0u;
  }
  return !std::isnan(scale);  // NaN never compares equal: not cached (and rejected anyway)
}

constexpr int kPlanCacheSize = 8;
struct PlanCacheEntry {
  bool used;
  FwdKey key;
  Plan plan;
};
thread_local PlanCacheEntry g_plan_cache[kPlanCacheSize];
thread_local int g_plan_cache_next = 0;

// The call's pointers into a plan made for other pointers with the same key.
void rebind_plan(Plan* P, const relattn_tensor* q, const relattn_tensor* k,
                 const relattn_tensor* v, const relattn_tensor* wK, const relattn_tensor* wV,
                 const relattn_tensor* t5_bias, const relattn_mask* mask,
                 const relattn_tensor* out) {
  FwdParams& p = P->p;
  p.q = q->data;
  p.k = k->data;
  p.v = v->data;
  p.o = out->data;
  p.wk = wK ? wK->data : nullptr;
  p.wv = wV ? wV->data : nullptr;
  p.t5_bias = t5_bias ? static_cast<const float*>(t5_bias->data) : nullptr;
  p.key_lens = mask ? mask->key_lens : nullptr;
  p.lse = nullptr;
}

// make_plan (with the T5 thresholds) through the cache.
int cached_fwd_plan(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                    const relattn_tensor* wK, const relattn_tensor* wV,
                    const relattn_tensor* t5_bias, const relattn_t5_params* t5, int32_t clip_k,
                    float scale, const relattn_mask* mask, const relattn_tensor* out,
                    Plan* plan) {
  FwdKey key;
  const bool keyed = q && k && v && out &&
                     make_fwd_key(q, k, v, wK, wV, t5_bias, t5, clip_k, scale, mask, out, &key);
  if (keyed) {
    for (int i = 0; i < kPlanCacheSize; ++i) {
      const PlanCacheEntry& e = g_plan_cache[i];
      if (e.used && std::memcmp(&e.key, &key, sizeof key) == 0) {
        *plan = e.plan;
        if (!plan->empty) rebind_plan(plan, q, k, v, wK, wV, t5_bias, mask, out);
        return RELATTN_OK;
      }
    }
  }
  const int st = make_plan(q, k, v, wK, wV, t5_bias, t5, clip_k, scale, mask, out, plan, true);
  if (st || !keyed) return st;
  PlanCacheEntry& e = g_plan_cache[g_plan_cache_next];
  g_plan_cache_next = (g_plan_cache_next + 1) % kPlanCacheSize;
  e.used = true;
  e.key = key;
  e.plan = *plan;
  return RELATTN_OK;
}

}  // namespace

extern "C" {

int relattn_fwd_lse(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                    const relattn_tensor* wK, const relattn_tensor* wV,
                    const relattn_tensor* t5_bias, const relattn_t5_params* t5, int32_t clip_k,
                    float scale, const relattn_mask* mask, relattn_tensor* out,
                    relattn_tensor* lse, void* stream) {
  g_last_error.clear();
  Plan plan;
  int st = cached_fwd_plan(q, k, v, wK, wV, t5_bias, t5, clip_k, scale, mask, out, &plan);
  if (st) return st;
  if ((st = check_lse(lse, q))) return st;
  return run_fwd_lse(plan, lse, stream);
}

int relattn_fwd_offset_bias_lse(const relattn_tensor* q, const relattn_tensor* k,
                                const relattn_tensor* v, const relattn_tensor* bias,
                                int32_t window, float scale, const relattn_mask* mask,
                                relattn_tensor* out, relattn_tensor* lse, void* stream) {
  g_last_error.clear();
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  Plan plan;
  int st = make_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out, &plan, true,
                     bias, window);
  if (st) return st;
  if ((st = check_lse(lse, q))) return st;
  return run_fwd_lse(plan, lse, stream);
}

int relattn_bwd_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                               const relattn_tensor* v, const relattn_tensor* wK,
                               const relattn_tensor* wV, const relattn_tensor* t5_bias,
                               const relattn_t5_params* t5, int32_t clip_k, float scale,
                               const relattn_mask* mask, const relattn_tensor* out,
                               const relattn_tensor* dout, const relattn_tensor* lse,
                               const relattn_tensor* dq, const relattn_tensor* dk,
                               const relattn_tensor* dv, const relattn_tensor* dwK,
                               const relattn_tensor* dwV, const relattn_tensor* dbias,
                               size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  BwdPlan plan;
  const int st = make_bwd_plan(q, k, v, wK, wV, t5_bias, t5, clip_k, scale, mask, out, dout, lse,
                               dq, dk, dv, dwK, dwV, dbias, &plan, true);
  if (st) return st;
  *bytes = plan.fwd.empty ? 0 : plan.ws_bytes;
  return RELATTN_OK;
}

int relattn_bwd(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                const relattn_tensor* wK, const relattn_tensor* wV,
                const relattn_tensor* t5_bias, const relattn_t5_params* t5, int32_t clip_k,
                float scale, const relattn_mask* mask, const relattn_tensor* out,
                const relattn_tensor* dout, const relattn_tensor* lse, relattn_tensor* dq,
                relattn_tensor* dk, relattn_tensor* dv, relattn_tensor* dwK, relattn_tensor* dwV,
                relattn_tensor* dbias, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  BwdPlan plan;
  const int st = make_bwd_plan(q, k, v, wK, wV, t5_bias, t5, clip_k, scale, mask, out, dout, lse,
                               dq, dk, dv, dwK, dwV, dbias, &plan, true);
  if (st) return st;
  return run_bwd(plan, wK, wV, t5_bias != nullptr && dbias != nullptr, workspace,
                 workspace_bytes, stream);
}

int relattn_bwd_offset_bias_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                           const relattn_tensor* v, const relattn_tensor* bias,
                                           int32_t window, float scale, const relattn_mask* mask,
                                           const relattn_tensor* out, const relattn_tensor* dout,
                                           const relattn_tensor* lse, const relattn_tensor* dq,
                                           const relattn_tensor* dk, const relattn_tensor* dv,
                                           const relattn_tensor* dbias, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  BwdPlan plan;
  const int st = make_bwd_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out,
                               dout, lse, dq, dk, dv, nullptr, nullptr, dbias, &plan, true, bias,
                               window);
  if (st) return st;
  *bytes = plan.fwd.empty ? 0 : plan.ws_bytes;
  return RELATTN_OK;
}

int relattn_bwd_offset_bias(const relattn_tensor* q, const relattn_tensor* k,
                            const relattn_tensor* v, const relattn_tensor* bias, int32_t window,
                            float scale, const relattn_mask* mask, const relattn_tensor* out,
                            const relattn_tensor* dout, const relattn_tensor* lse,
                            relattn_tensor* dq, relattn_tensor* dk, relattn_tensor* dv,
                            relattn_tensor* dbias, void* workspace, size_t workspace_bytes,
                            void* stream) {
  g_last_error.clear();
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  BwdPlan plan;
  const int st = make_bwd_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out,
                               dout, lse, dq, dk, dv, nullptr, nullptr, dbias, &plan, true, bias,
                               window);
  if (st) return st;
  return run_bwd(plan, nullptr, nullptr, dbias != nullptr, workspace, workspace_bytes, stream);
}


int relattn_validate(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                     const relattn_tensor* wK, const relattn_tensor* wV,
                     const relattn_tensor* t5_bias, const relattn_t5_params* t5,
                     int32_t clip_k, float scale, const relattn_mask* mask,
                     const relattn_tensor* out) {
  g_last_error.clear();
  Plan plan;
  return make_plan(q, k, v, wK, wV, t5_bias, t5, clip_k, scale, mask, out, &plan, false);
}

int relattn_fwd(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                const relattn_tensor* wK, const relattn_tensor* wV,
                const relattn_tensor* t5_bias, const relattn_t5_params* t5, int32_t clip_k,
                float scale, const relattn_mask* mask, relattn_tensor* out, void* stream) {
  g_last_error.clear();
  Plan plan;
  const int st = cached_fwd_plan(q, k, v, wK, wV, t5_bias, t5, clip_k, scale, mask, out, &plan);
  if (st) return st;
  return run_fwd(plan, stream);
}

int relattn_validate_offset_bias(const relattn_tensor* q, const relattn_tensor* k,
                                 const relattn_tensor* v, const relattn_tensor* bias,
                                 int32_t window, float scale, const relattn_mask* mask,
                                 const relattn_tensor* out) {
  g_last_error.clear();
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  Plan plan;
  return make_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out, &plan, false,
                   bias, window);
}

int relattn_fwd_offset_bias(const relattn_tensor* q, const relattn_tensor* k,
                            const relattn_tensor* v, const relattn_tensor* bias, int32_t window,
                            float scale, const relattn_mask* mask, relattn_tensor* out,
                            void* stream) {
  g_last_error.clear();
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  Plan plan;
  int st = make_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out, &plan, true,
                     bias, window);
  if (st) return st;
  return run_fwd(plan, stream);
}

int relattn_validate_xl(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                        const relattn_tensor* R, const relattn_tensor* u, const relattn_tensor* vb,
                        int32_t window, float scale, const relattn_mask* mask,
                        const relattn_tensor* out) {
  g_last_error.clear();
  if (!R || !u || !vb) return fail(RELATTN_ERR_INVALID_ARGUMENT, "R, u and v are required");
  Plan plan;
  return make_plan(q, k, v, R, nullptr, nullptr, nullptr, window, scale, mask, out, &plan, false,
                   nullptr, 0, u, vb);
}

int relattn_fwd_xl(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                   const relattn_tensor* R, const relattn_tensor* u, const relattn_tensor* vb,
                   int32_t window, float scale, const relattn_mask* mask, relattn_tensor* out,
                   void* stream) {
  g_last_error.clear();
  if (!R || !u || !vb) return fail(RELATTN_ERR_INVALID_ARGUMENT, "R, u and v are required");
  Plan plan;
  int st = make_plan(q, k, v, R, nullptr, nullptr, nullptr, window, scale, mask, out, &plan, true,
                     nullptr, 0, u, vb);
  if (st) return st;
  return run_fwd(plan, stream);
}

int relattn_fwd_xl_lse(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                       const relattn_tensor* R, const relattn_tensor* u, const relattn_tensor* vb,
                       int32_t window, float scale, const relattn_mask* mask, relattn_tensor* out,
                       relattn_tensor* lse, void* stream) {
  g_last_error.clear();
  if (!R || !u || !vb) return fail(RELATTN_ERR_INVALID_ARGUMENT, "R, u and v are required");
  Plan plan;
  int st = make_plan(q, k, v, R, nullptr, nullptr, nullptr, window, scale, mask, out, &plan, true,
                     nullptr, 0, u, vb);
  if (st) return st;
  if ((st = check_lse(lse, q))) return st;
  return run_fwd_lse(plan, lse, stream);
}

int relattn_bwd_xl_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                  const relattn_tensor* v, const relattn_tensor* R,
                                  const relattn_tensor* u, const relattn_tensor* vb,
                                  int32_t window, float scale, const relattn_mask* mask,
                                  const relattn_tensor* out, const relattn_tensor* dout,
                                  const relattn_tensor* lse, const relattn_tensor* dq,
                                  const relattn_tensor* dk, const relattn_tensor* dv,
                                  const relattn_tensor* dR, const relattn_tensor* du,
                                  const relattn_tensor* dvb, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (!R || !u || !vb) return fail(RELATTN_ERR_INVALID_ARGUMENT, "R, u and v are required");
  BwdPlan plan;
  const int st = make_bwd_plan(q, k, v, R, nullptr, nullptr, nullptr, window, scale, mask, out,
                               dout, lse, dq, dk, dv, dR, nullptr, nullptr, &plan, true, nullptr,
                               0, 0, nullptr, u, vb, du, dvb);
  if (st) return st;
  *bytes = plan.fwd.empty ? 0 : plan.ws_bytes;
  return RELATTN_OK;
}

int relattn_bwd_xl(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                   const relattn_tensor* R, const relattn_tensor* u, const relattn_tensor* vb,
                   int32_t window, float scale, const relattn_mask* mask,
                   const relattn_tensor* out, const relattn_tensor* dout,
                   const relattn_tensor* lse, relattn_tensor* dq, relattn_tensor* dk,
                   relattn_tensor* dv, relattn_tensor* dR, relattn_tensor* du,
                   relattn_tensor* dvb, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!R || !u || !vb) return fail(RELATTN_ERR_INVALID_ARGUMENT, "R, u and v are required");
  BwdPlan plan;
  const int st = make_bwd_plan(q, k, v, R, nullptr, nullptr, nullptr, window, scale, mask, out,
                               dout, lse, dq, dk, dv, dR, nullptr, nullptr, &plan, true, nullptr,
                               0, 0, nullptr, u, vb, du, dvb);
  if (st) return st;
  return run_bwd(plan, R, nullptr, false, workspace, workspace_bytes, stream);
}

int relattn_fwd_grid_bias_lse(const relattn_tensor* q, const relattn_tensor* k,
                              const relattn_tensor* v, const relattn_tensor* bias,
                              int32_t window_side, float scale, const relattn_mask* mask,
                              relattn_tensor* out, relattn_tensor* lse, void* stream) {
  g_last_error.clear();
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  if (window_side < 1) return fail(RELATTN_ERR_INVALID_ARGUMENT, "window side M must be >= 1");
  Plan plan;
  int st = make_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out, &plan, true,
                     bias, 0, nullptr, nullptr, window_side);
  if (st) return st;
  if ((st = check_lse(lse, q))) return st;
  return run_fwd_lse(plan, lse, stream);
}

int relattn_bwd_grid_bias_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                         const relattn_tensor* v, const relattn_tensor* bias,
                                         int32_t window_side, float scale,
                                         const relattn_mask* mask, const relattn_tensor* out,
                                         const relattn_tensor* dout, const relattn_tensor* lse,
                                         const relattn_tensor* dq, const relattn_tensor* dk,
                                         const relattn_tensor* dv, const relattn_tensor* dbias,
                                         size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  if (window_side < 1) return fail(RELATTN_ERR_INVALID_ARGUMENT, "window side M must be >= 1");
  BwdPlan plan;
  const int st = make_bwd_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out,
                               dout, lse, dq, dk, dv, nullptr, nullptr, dbias, &plan, true, bias,
                               0, window_side);
  if (st) return st;
  *bytes = plan.fwd.empty ? 0 : plan.ws_bytes;
  return RELATTN_OK;
}

int relattn_bwd_grid_bias(const relattn_tensor* q, const relattn_tensor* k,
                          const relattn_tensor* v, const relattn_tensor* bias,
                          int32_t window_side, float scale, const relattn_mask* mask,
                          const relattn_tensor* out, const relattn_tensor* dout,
                          const relattn_tensor* lse, relattn_tensor* dq, relattn_tensor* dk,
                          relattn_tensor* dv, relattn_tensor* dbias, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  if (window_side < 1) return fail(RELATTN_ERR_INVALID_ARGUMENT, "window side M must be >= 1");
  BwdPlan plan;
  const int st = make_bwd_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out,
                               dout, lse, dq, dk, dv, nullptr, nullptr, dbias, &plan, true, bias,
                               0, window_side);
  if (st) return st;
  return run_bwd(plan, nullptr, nullptr, dbias != nullptr, workspace, workspace_bytes, stream);
}


int relattn_validate_grid_bias(const relattn_tensor* q, const relattn_tensor* k,
                               const relattn_tensor* v, const relattn_tensor* bias,
                               int32_t window_side, float scale, const relattn_mask* mask,
                               const relattn_tensor* out) {
  g_last_error.clear();
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  if (window_side < 1) return fail(RELATTN_ERR_INVALID_ARGUMENT, "window side M must be >= 1");
  Plan plan;
  return make_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out, &plan, false,
                   bias, 0, nullptr, nullptr, window_side);
}

int relattn_fwd_grid_bias(const relattn_tensor* q, const relattn_tensor* k,
                          const relattn_tensor* v, const relattn_tensor* bias,
                          int32_t window_side, float scale, const relattn_mask* mask,
                          relattn_tensor* out, void* stream) {
  g_last_error.clear();
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  if (window_side < 1) return fail(RELATTN_ERR_INVALID_ARGUMENT, "window side M must be >= 1");
  Plan plan;
  int st = make_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out, &plan, true,
                     bias, 0, nullptr, nullptr, window_side);
  if (st) return st;
  return run_fwd(plan, stream);
}

int relattn_validate_edge_bias(const relattn_tensor* q, const relattn_tensor* k,
                               const relattn_tensor* v, const relattn_tensor* labels,
                               const relattn_tensor* bias, float scale, const relattn_mask* mask,
                               const relattn_tensor* out) {
  g_last_error.clear();
  if (!labels) return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels is NULL");
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  Plan plan;
  return make_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out, &plan, false,
                   bias, 0, nullptr, nullptr, 0, labels);
}

int relattn_fwd_edge_bias(const relattn_tensor* q, const relattn_tensor* k,
                          const relattn_tensor* v, const relattn_tensor* labels,
                          const relattn_tensor* bias, float scale, const relattn_mask* mask,
                          relattn_tensor* out, void* stream) {
  g_last_error.clear();
  if (!labels) return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels is NULL");
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  Plan plan;
  int st = make_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out, &plan, true,
                     bias, 0, nullptr, nullptr, 0, labels);
  if (st) return st;
  return run_fwd(plan, stream);
}

int relattn_fwd_edge_bias_lse(const relattn_tensor* q, const relattn_tensor* k,
                              const relattn_tensor* v, const relattn_tensor* labels,
                              const relattn_tensor* bias, float scale, const relattn_mask* mask,
                              relattn_tensor* out, relattn_tensor* lse, void* stream) {
  g_last_error.clear();
  if (!labels) return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels is NULL");
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  Plan plan;
  int st = make_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out, &plan, true,
                     bias, 0, nullptr, nullptr, 0, labels);
  if (st) return st;
  if ((st = check_lse(lse, q))) return st;
  return run_fwd_lse(plan, lse, stream);
}

int relattn_bwd_edge_bias_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                         const relattn_tensor* v, const relattn_tensor* labels,
                                         const relattn_tensor* bias, float scale,
                                         const relattn_mask* mask, const relattn_tensor* out,
                                         const relattn_tensor* dout, const relattn_tensor* lse,
                                         const relattn_tensor* dq, const relattn_tensor* dk,
                                         const relattn_tensor* dv, const relattn_tensor* dbias,
                                         size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (!labels) return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels is NULL");
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  BwdPlan plan;
  const int st = make_bwd_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out,
                               dout, lse, dq, dk, dv, nullptr, nullptr, dbias, &plan, true, bias,
                               0, 0, labels);
  if (st) return st;
  *bytes = plan.fwd.empty ? 0 : plan.ws_bytes;
  return RELATTN_OK;
}

int relattn_bwd_edge_bias(const relattn_tensor* q, const relattn_tensor* k,
                          const relattn_tensor* v, const relattn_tensor* labels,
                          const relattn_tensor* bias, float scale, const relattn_mask* mask,
                          const relattn_tensor* out, const relattn_tensor* dout,
                          const relattn_tensor* lse, relattn_tensor* dq, relattn_tensor* dk,
                          relattn_tensor* dv, relattn_tensor* dbias, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!labels) return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels is NULL");
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  BwdPlan plan;
  const int st = make_bwd_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, mask, out,
                               dout, lse, dq, dk, dv, nullptr, nullptr, dbias, &plan, true, bias,
                               0, 0, labels);
  if (st) return st;
  return run_bwd(plan, nullptr, nullptr, dbias != nullptr, workspace, workspace_bytes, stream);
}

int relattn_fwd_edge_tables_lse(const relattn_tensor* q, const relattn_tensor* k,
                                const relattn_tensor* v, const relattn_tensor* labels,
                                const relattn_tensor* wK, const relattn_tensor* wV, float scale,
                                const relattn_mask* mask, relattn_tensor* out,
                                relattn_tensor* lse, void* stream) {
  g_last_error.clear();
  if (!labels) return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels is NULL");
  Plan plan;
  int st = make_plan(q, k, v, wK, wV, nullptr, nullptr, 0, scale, mask, out, &plan, true, nullptr,
                     0, nullptr, nullptr, 0, labels);
  if (st) return st;
  if ((st = check_lse(lse, q))) return st;
  return run_fwd_lse(plan, lse, stream);
}

int relattn_bwd_edge_tables_workspace_size(
    const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
    const relattn_tensor* labels, const relattn_tensor* wK, const relattn_tensor* wV, float scale,
    const relattn_mask* mask, const relattn_tensor* out, const relattn_tensor* dout,
    const relattn_tensor* lse, const relattn_tensor* dq, const relattn_tensor* dk,
    const relattn_tensor* dv, const relattn_tensor* dwK, const relattn_tensor* dwV,
    size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (!labels) return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels is NULL");
  BwdPlan plan;
  const int st = make_bwd_plan(q, k, v, wK, wV, nullptr, nullptr, 0, scale, mask, out, dout, lse,
                               dq, dk, dv, dwK, dwV, nullptr, &plan, true, nullptr, 0, 0, labels);
  if (st) return st;
  *bytes = plan.fwd.empty ? 0 : plan.ws_bytes;
  return RELATTN_OK;
}

int relattn_bwd_edge_tables(const relattn_tensor* q, const relattn_tensor* k,
                            const relattn_tensor* v, const relattn_tensor* labels,
                            const relattn_tensor* wK, const relattn_tensor* wV, float scale,
                            const relattn_mask* mask, const relattn_tensor* out,
                            const relattn_tensor* dout, const relattn_tensor* lse,
                            relattn_tensor* dq, relattn_tensor* dk, relattn_tensor* dv,
                            relattn_tensor* dwK, relattn_tensor* dwV, void* workspace,
                            size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!labels) return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels is NULL");
  BwdPlan plan;
  const int st = make_bwd_plan(q, k, v, wK, wV, nullptr, nullptr, 0, scale, mask, out, dout, lse,
                               dq, dk, dv, dwK, dwV, nullptr, &plan, true, nullptr, 0, 0, labels);
  if (st) return st;
  return run_bwd(plan, wK, wV, false, workspace, workspace_bytes, stream);
}

int relattn_validate_edge_tables(const relattn_tensor* q, const relattn_tensor* k,
                                 const relattn_tensor* v, const relattn_tensor* labels,
                                 const relattn_tensor* wK, const relattn_tensor* wV, float scale,
                                 const relattn_mask* mask, const relattn_tensor* out) {
  g_last_error.clear();
  if (!labels) return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels is NULL");
  Plan plan;
  return make_plan(q, k, v, wK, wV, nullptr, nullptr, 0, scale, mask, out, &plan, false, nullptr,
                   0, nullptr, nullptr, 0, labels);
}

int relattn_fwd_edge_tables(const relattn_tensor* q, const relattn_tensor* k,
                            const relattn_tensor* v, const relattn_tensor* labels,
                            const relattn_tensor* wK, const relattn_tensor* wV, float scale,
                            const relattn_mask* mask, relattn_tensor* out, void* stream) {
  g_last_error.clear();
  if (!labels) return fail(RELATTN_ERR_INVALID_ARGUMENT, "labels is NULL");
  Plan plan;
  int st = make_plan(q, k, v, wK, wV, nullptr, nullptr, 0, scale, mask, out, &plan, true, nullptr,
                     0, nullptr, nullptr, 0, labels);
  if (st) return st;
  return run_fwd(plan, stream);
}

int relattn_debug_indices(int32_t n, int32_t clip_k, const relattn_t5_params* t5,
                          int32_t* out_dev, void* stream) {
  g_last_error.clear();
  if (n < 1 || n > kMaxSeq) return fail(RELATTN_ERR_INVALID_ARGUMENT, "n must be in [1, 2^30]");
  if (!out_dev) return fail(RELATTN_ERR_INVALID_ARGUMENT, "out_dev is NULL");
  if (reinterpret_cast<uintptr_t>(out_dev) & 3u)
    return fail(RELATTN_ERR_INVALID_ARGUMENT, "out_dev is not 4-byte aligned");
  if (!t5 && clip_k < 0) return fail(RELATTN_ERR_INVALID_ARGUMENT, "clip_k must be >= 0");
  T5Buckets tb = {};
  int st;
  if (t5 && (st = check_t5(t5, &tb))) return st;
  if ((st = check_device())) return st;
  const int e = relattn::launch_debug_indices(n, clip_k, t5 ? &tb : nullptr, out_dev, stream);
  if (e != (int)hipSuccess)
    return fail(RELATTN_ERR_LAUNCH_FAILED, "launch failed: %s",
                hipGetErrorString((hipError_t)e));
  return RELATTN_OK;
}

int relattn_decode_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                  const relattn_tensor* v, const relattn_tensor* wK,
                                  const relattn_tensor* wV, const relattn_tensor* t5_bias,
                                  const relattn_t5_params* t5, int32_t clip_k, float scale,
                                  const relattn_tensor* out, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  DecPlan plan;
  const int st = make_dec_plan(q, k, v, wK, wV, t5_bias, t5, clip_k, scale, out, &plan, false);
  if (st) return st;
  *bytes = plan.empty ? 0 : plan.ws_bytes;
  return RELATTN_OK;
}

int relattn_decode(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                   const relattn_tensor* wK, const relattn_tensor* wV,
                   const relattn_tensor* t5_bias, const relattn_t5_params* t5, int32_t clip_k,
                   float scale, const int32_t* cache_lens, relattn_tensor* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  DecPlan plan;
  int st = make_dec_plan(q, k, v, wK, wV, t5_bias, t5, clip_k, scale, out, &plan, true);
  if (st) return st;
  return run_decode(plan, cache_lens, workspace, workspace_bytes, stream);
}

int relattn_decode_noalloc(const relattn_tensor* q, const relattn_tensor* k,
                           const relattn_tensor* v, const relattn_tensor* wK,
                           const relattn_tensor* wV, const relattn_tensor* t5_bias,
                           const relattn_t5_params* t5, int32_t clip_k, float scale,
                           const int32_t* cache_lens, relattn_tensor* out, void* stream) {
  g_last_error.clear();
  DecPlan plan;
  int st = make_dec_plan(q, k, v, wK, wV, t5_bias, t5, clip_k, scale, out, &plan, true);
  if (st) return st;
  if (!plan.empty && plan.ws_bytes > kScratchBytes)
    return fail(RELATTN_ERR_UNSUPPORTED,
                "these shapes need %zu bytes of workspace; the static scratch holds %zu",
                plan.ws_bytes, kScratchBytes);
  if ((st = check_device())) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return run_decode(plan, cache_lens, ws, kScratchBytes, stream);
}

int relattn_decode_xl_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                     const relattn_tensor* v, const relattn_tensor* R,
                                     const relattn_tensor* u, const relattn_tensor* vb,
                                     int32_t window, float scale, const relattn_tensor* out,
                                     size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (!R || !u || !vb) return fail(RELATTN_ERR_INVALID_ARGUMENT, "R, u and v must be given");
  DecPlan plan;
  const int st = make_dec_plan(q, k, v, R, nullptr, nullptr, nullptr, window, scale, out, &plan,
                               false, nullptr, 0, u, vb);
  if (st) return st;
  *bytes = plan.empty ? 0 : plan.ws_bytes;
  return RELATTN_OK;
}

int relattn_decode_xl(const relattn_tensor* q, const relattn_tensor* k, const relattn_tensor* v,
                      const relattn_tensor* R, const relattn_tensor* u, const relattn_tensor* vb,
                      int32_t window, float scale, const int32_t* cache_lens, relattn_tensor* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!R || !u || !vb) return fail(RELATTN_ERR_INVALID_ARGUMENT, "R, u and v must be given");
  DecPlan plan;
  int st = make_dec_plan(q, k, v, R, nullptr, nullptr, nullptr, window, scale, out, &plan, true,
                         nullptr, 0, u, vb);
  if (st) return st;
  return run_decode(plan, cache_lens, workspace, workspace_bytes, stream);
}

int relattn_decode_offset_bias_workspace_size(const relattn_tensor* q, const relattn_tensor* k,
                                              const relattn_tensor* v, const relattn_tensor* bias,
                                              int32_t window, float scale,
                                              const relattn_tensor* out, size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  DecPlan plan;
  const int st = make_dec_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, out, &plan,
                               false, bias, window);
  if (st) return st;
  *bytes = plan.empty ? 0 : plan.ws_bytes;
  return RELATTN_OK;
}

int relattn_decode_offset_bias(const relattn_tensor* q, const relattn_tensor* k,
                               const relattn_tensor* v, const relattn_tensor* bias, int32_t window,
                               float scale, const int32_t* cache_lens, relattn_tensor* out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!bias) return fail(RELATTN_ERR_INVALID_ARGUMENT, "bias is NULL");
  DecPlan plan;
  int st = make_dec_plan(q, k, v, nullptr, nullptr, nullptr, nullptr, 0, scale, out, &plan, true,
                         bias, window);
  if (st) return st;
  return run_decode(plan, cache_lens, workspace, workspace_bytes, stream);
}

const char* relattn_strerror(int status) {
  switch (status) {
    case RELATTN_OK: return "ok";
    case RELATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case RELATTN_ERR_UNSUPPORTED: return "unsupported";
    case RELATTN_ERR_NO_DEVICE: return "no device";
    case RELATTN_ERR_LAUNCH_FAILED: return "launch failed";
  }
  return "unknown status";
}

const char* relattn_last_error(void) { return g_last_error.c_str(); }

int relattn_version(void) { return RELATTN_VERSION; }

}  // extern "C"
