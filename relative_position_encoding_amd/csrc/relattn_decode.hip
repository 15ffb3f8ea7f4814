// Incremental decoding for gfx950: the newest Tq positions of each sequence
// attend over its key/value cache ("Self-Attention with Relative Position
// Representations", section 3.4, Eq. 3 and Eq. 4 with r = clip(j - i, k);
// T5 section of "Relative position embeddings" for the bias variant).  Query
// t of batch b sits at position i = len_b - Tq + t and sees keys j <= i.
//
// One decoding step reads the whole cache once and does little arithmetic per
// byte, so the work is split into chunks of the cache that stream from HBM in
// parallel:
//   decode_partial_kernel  one workgroup per (query row, chunk of keys): the
//       chunk's logits e_j = scale * q . (k_j + a^K_ij) in log2 units (T5: the
//       bucketed bias instead of a^K; or the entry of a table by clipped
//       offset, e.g. ALiBi; Transformer-XL: (q + u).k_j + (q + v).R_{i-j} with the
//       position table's row of each key requested with its K row), its max
//       m_c, the sum l_c of 2^(e_j - m_c)
//       and the partial output O_c = sum_j 2^(e_j - m_c) v_j.  Each K and V row
//       is read by LPR lanes with 16-byte loads (coalesced rows, every load of
//       a lane issued before the first use); a dot product is summed over the
//       LPR lanes of its row.  The raw logits of keys whose label holds them
//       alone (offsets -k < j - i <= 0) are kept for the value term.
//   decode_combine_kernel  one workgroup per query row: m = max m_c,
//       l = sum l_c 2^(m_c - m), O = sum O_c 2^(m_c - m); the value term adds
//       2^(e_j - m) a^V for each single-key label and the remaining weight
//       l - sum of those for label -k; z = O / l.  Chunk factors and label
//       weights are computed in parallel and staged in LDS; the column sums
//       are split over groups of threads so that their loads are independent.
//       (A separate kernel: handing partial results from one workgroup to
//       another inside one launch needs device-scope fences, which write back
//       and invalidate the XCDs' L2 caches and cost far more than a launch.)
#include <hip/hip_runtime.h>

#include <type_traits>

#include "relattn_device.h"
#include "relattn_internal.h"

namespace relattn {
namespace {

constexpr int kDecThreads = 256;
// rows with at most this many splits and single-key labels take the combine
// path that issues every load at once
constexpr int kFastChunks = 8;
constexpr int kFastLabels = 64;

template <bool BF16>
struct Frag;  // 16 bytes of a row
template <>
struct Frag<true> {
  using V = bf16x8;
  static constexpr int N = 8;
};
template <>
struct Frag<false> {
  using V = f32x4;
  static constexpr int N = 4;
};

template <bool BF16>
__device__ __forceinline__ typename Frag<BF16>::V load_frag(const void* base, int64_t elem) {
  using V = typename Frag<BF16>::V;
  return *reinterpret_cast<const V*>(static_cast<const char*>(base) + elem * (BF16 ? 2 : 4));
}

// Sum over the W consecutive lanes that share a row (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = W / 2; o > 0; o /= 2) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o /= 2) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o /= 2) x += __shfl_xor(x, o);
  return x;
}

// Position of query row `row` = (b * H + h) * Tq + t, and its batch and head.
struct RowPos {
  int b, h, t, i;
};
__device__ __forceinline__ RowPos row_pos(const DecParams& p, int row) {
  RowPos r;
  r.t = row % p.Tq;
  const int bh = row / p.Tq;
  r.b = bh / p.H;
  r.h = bh - r.b * p.H;
  const int len = p.cache_lens ? min(max(p.cache_lens[r.b], 0), p.L) : p.L;
  r.i = len - p.Tq + r.t;
  return r;
}

// Waves per SIMD the register budget is sized for: four, except Transformer-XL,
// whose position-table rows (requested with the K rows) would spill there.
template <int MODE>
constexpr int dec_waves_per_eu() {
  return MODE == kRelXL ? 2 : 4;
}

template <int D, bool BF16, int MODE, bool HAS_WK, bool HAS_WV, bool DIRECT>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(
    dec_waves_per_eu<MODE>()))) void decode_kernel(
    const DecParams p) {
  using V = typename Frag<BF16>::V;
  using T = std::conditional_t<BF16, __bf16, float>;
  constexpr int EPL = Frag<BF16>::N;           // elements per 16-byte load
  constexpr int LPR = D / EPL;                 // lanes per row
  constexpr int RPP = kDecThreads / LPR;       // rows per pass
  constexpr int CH = dec_chunk(BF16 ? 2 : 4, D);
  constexpr int NP = CH / RPP;                 // passes (8)
  constexpr int NG = kDecThreads / D;          // column groups of the value term
  static_assert(LPR >= 1 && LPR <= 64 && NP * RPP == CH, "chunk geometry");
  constexpr bool SHAW = MODE == kRelShaw;
  constexpr bool T5 = MODE == kRelT5;
  constexpr bool XLD = MODE == kRelXL;  // Transformer-XL: wk is the position table R
  constexpr bool VT = SHAW && HAS_WV;
  __shared__ float s_e[CH];
  __shared__ float s_red[8];
  __shared__ float s_acc[RPP * D];
  __shared__ float s_band[DIRECT && VT ? kDirectBand : 1];

  const int row = blockIdx.x, split = blockIdx.y;
  const RowPos rp = row_pos(p, row);
  const int i = rp.i, b = rp.b, h = rp.h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (i < 0) {  // no visible key: zeros (written here when this workgroup owns the row)
    if (DIRECT && tid < D)
      reinterpret_cast<T*>(p.o)[b * p.o_sb + h * p.o_sh + rp.t * p.o_st + tid] = (T)0.f;
    return;
  }
  // this workgroup's chunks of the row (the same for the whole workgroup)
  const int cb = split * p.cps, ce = min(cb + p.cps, i / CH + 1);
  if (cb >= ce) return;
  const int part = tid % LPR, rs = tid / LPR;
  const int c0 = part * EPL;  // first column of this lane's fragment

  float qf[EPL];
  {
    const V x = load_frag<BF16>(p.q, b * p.q_sb + h * p.q_sh + rp.t * p.q_st + c0);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[e] = (float)x[e];
  }
  // Transformer-XL: q + v for the position term, q + u for the content term,
  // each rounded once to the input dtype (as the forward does)
  float qv[XLD ? EPL : 1];
  if constexpr (XLD) {
    const V xu = load_frag<BF16>(p.xl_u, h * p.xl_u_sh + c0);
    const V xv = load_frag<BF16>(p.xl_v, h * p.xl_v_sh + c0);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      qv[e] = (float)(T)(qf[e] + (float)xv[e]);
      qf[e] = (float)(T)(qf[e] + (float)xu[e]);
    }
  }
  const int64_t kb = b * p.k_sb + h * p.k_sh, vb = b * p.v_sb + h * p.v_sh;

  // relative logit of every key at offset <= -k (label row 0)
  float far = 0.f;
  if constexpr (SHAW && HAS_WK) {
    const V w = load_frag<BF16>(p.wk, h * p.wk_sh + c0);
    float d0 = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) d0 = fmaf(qf[e], (float)w[e], d0);
    far = group_sum<LPR>(d0) * p.scale_log2;
  }

  // online softmax over the chunks: running max and sum, this lane's columns
  float m_run = kNegInf, l_run = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int c = cb; c < ce; ++c) {
    const int j0 = c * CH, j1 = min(j0 + CH, i + 1);
    // every K and V fragment of this lane for the chunk, requested before the
    // first use; rows past the last visible key read that key again (finite,
    // weighted 0)
    V kf[NP], vf[NP];
#pragma unroll
    for (int it = 0; it < NP; ++it) {
      const int j = min(j0 + rs + it * RPP, j1 - 1);
      kf[it] = load_frag<BF16>(p.k, kb + j * p.k_sn + c0);
    }
#pragma unroll
    for (int it = 0; it < NP; ++it) {
      const int j = min(j0 + rs + it * RPP, j1 - 1);
      vf[it] = load_frag<BF16>(p.v, vb + j * p.v_sn + c0);
    }
    // Transformer-XL: each key's position-table row, distance i - j clamped to
    // the window (row clip + distance)
    V rf[XLD ? NP : 1];
    if constexpr (XLD) {
#pragma unroll
      for (int it = 0; it < NP; ++it) {
        const int j = min(j0 + rs + it * RPP, j1 - 1);
        const int dist = min(i - j, p.clip);
        rf[it] = load_frag<BF16>(p.wk, h * p.wk_sh + (p.clip + dist) * p.wk_sr + c0);
      }
    }
    // logits, log2 units
#pragma unroll
    for (int it = 0; it < NP; ++it) {
      const int r = rs + it * RPP;
      const bool valid = j0 + r < j1;
      const int j = min(j0 + r, j1 - 1);
      const int delta = j - i;  // <= 0
      float x[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = (float)kf[it][e];
      float rel = 0.f;
      if constexpr (SHAW && HAS_WK) {
        if (delta > -p.clip) {
          // inside the window: a^K of this key's own label joins k_j (Eq. 4)
          const V w = load_frag<BF16>(p.wk, h * p.wk_sh + (delta + p.clip) * p.wk_sr + c0);
#pragma unroll
          for (int e = 0; e < EPL; ++e) x[e] += (float)w[e];
        } else {
          rel = far;
        }
      }
      if constexpr (T5) {
        // T5 bucket, or the entry of a table by clipped offset
        const int entry = p.ob ? min(max(delta, -p.ob_w), p.ob_w) + p.ob_w : t5_bucket(delta, p.t5);
        rel = kLog2e * p.t5_bias[entry * p.tb_sb + h * p.tb_sh];
      }
      float dot = 0.f;
      if constexpr (XLD) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = fmaf(qv[e], (float)rf[it][e], dot);
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = fmaf(qf[e], x[e], dot);
      dot = group_sum<LPR>(dot);
      const float lg = valid ? fmaf(dot, p.scale_log2, rel) : kNegInf;
      if (part == 0) {
        s_e[r] = lg;
        if constexpr (VT) {
          if (valid && delta > -p.clip) {
            if constexpr (DIRECT) s_band[delta + p.nband - 1] = lg;
            else p.ws_band[(int64_t)row * p.nband + delta + p.nband - 1] = lg;
          }
        }
      }
    }
    __syncthreads();
    // chunk max; the running state then moves to the new max
    float mc = kNegInf;
    for (int x = tid; x < CH; x += kDecThreads) mc = fmaxf(mc, s_e[x]);
    mc = wave_max(mc);
    if (lane == 0) s_red[wave] = mc;
    __syncthreads();
    const float m_new = fmaxf(m_run, fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3])));
    const float sc = fast_exp2(m_run - m_new);  // 0 before the first chunk
    float lc = 0.f;
    for (int x = tid; x < CH; x += kDecThreads) {
      const float pv = fast_exp2(s_e[x] - m_new);  // 0 for the rows past the last key
      s_e[x] = pv;
      lc += pv;
    }
    lc = wave_sum(lc);
    if (lane == 0) s_red[4 + wave] = lc;
    __syncthreads();
    l_run = fmaf(l_run, sc, (s_red[4] + s_red[5]) + (s_red[6] + s_red[7]));
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= sc;
#pragma unroll
    for (int it = 0; it < NP; ++it) {
      const float pv = s_e[rs + it * RPP];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pv, (float)vf[it][e], acc[e]);
    }
    __syncthreads();  // s_e and s_red are rewritten by the next chunk
  }

  // this workgroup's output columns: the lanes' sums over their rows, summed
  // over the row groups through LDS
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_acc[rs * D + c0 + e] = acc[e];
  __syncthreads();
  if constexpr (!DIRECT) {
    const int64_t slot = (int64_t)row * p.nsp + split;
    for (int dim = tid; dim < D; dim += kDecThreads) {
      float o = 0.f;
      for (int g = 0; g < RPP; ++g) o += s_acc[g * D + dim];
      p.ws_o[slot * D + dim] = o;
    }
    if (tid == 0) {
      p.ws_ml[2 * slot] = m_run;
      p.ws_ml[2 * slot + 1] = l_run;
    }
  } else {
    // The workgroup holds the whole row: value term and output here.  Thread
    // (dim, grp) sums column dim over the row groups grp, grp + NG, ... and
    // over the single-key labels grp, grp + NG, ...
    const int dim = tid % D, grp = tid / D;
    float o = 0.f;
    for (int g = grp; g < RPP; g += NG) o += s_acc[g * D + dim];
    float sbp = 0.f;  // this group's share of the single-key weights
    float w0 = 0.f;
    if constexpr (VT) {
      const T* wvh = reinterpret_cast<const T*>(p.wv) + h * p.wv_sh;
      const int lo = max(1 - p.nband, -i);  // lowest offset with a key
      for (int x = grp; x < 1 - lo; x += NG) {
        const float w = fast_exp2(s_band[lo + x + p.nband - 1] - m_run);
        sbp += w;
        o = fmaf(w, (float)wvh[(lo + x + p.clip) * p.wv_sr + dim], o);
      }
      w0 = (float)wvh[dim];  // label -k
    }
    __syncthreads();  // s_acc and s_e are reused for the group sums
    s_acc[tid] = o;
    if (dim == 0) s_e[grp] = sbp;
    __syncthreads();
    if (tid < D) {
      float z = 0.f, sb = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        z += s_acc[g * D + tid];
        sb += s_e[g];
      }
      if constexpr (VT) z = fmaf(fmaxf(l_run - sb, 0.f), w0, z);
      reinterpret_cast<T*>(p.o)[b * p.o_sb + h * p.o_sh + rp.t * p.o_st + tid] = (T)(z / l_run);
    }
  }
}

// Sum (or max) over the 256 threads of the workgroup; `slot` picks a private
// group of LDS words so that consecutive reductions need no extra barrier.
__device__ __forceinline__ float block_sum(float x, float* red, int slot) {
  x = wave_sum(x);
  if ((threadIdx.x & 63) == 0) red[4 * slot + (threadIdx.x >> 6)] = x;
  __syncthreads();
  return (red[4 * slot] + red[4 * slot + 1]) + (red[4 * slot + 2] + red[4 * slot + 3]);
}
__device__ __forceinline__ float block_max(float x, float* red, int slot) {
  x = wave_max(x);
  if ((threadIdx.x & 63) == 0) red[4 * slot + (threadIdx.x >> 6)] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[4 * slot], red[4 * slot + 1]), fmaxf(red[4 * slot + 2], red[4 * slot + 3]));
}

template <int D, bool BF16, int MODE, bool HAS_WV>
__global__ __launch_bounds__(kDecThreads) void decode_combine_kernel(const DecParams p) {
  using T = std::conditional_t<BF16, __bf16, float>;
  constexpr int CH = dec_chunk(BF16 ? 2 : 4, D);
  constexpr int NG = kDecThreads / D;  // column groups
  constexpr int TILE = 1024;           // chunk factors / label weights staged at a time
  constexpr bool VT = MODE == kRelShaw && HAS_WV;
  __shared__ float s_f[TILE];
  __shared__ float s_red[12];
  __shared__ float s_o[kDecThreads];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int dim = tid % D, grp = tid / D;
  const float* ml = p.ws_ml + (int64_t)row * p.nsp * 2;
  const float* po = p.ws_o + (int64_t)row * p.nsp * D;
  const T* wv = reinterpret_cast<const T*>(p.wv);
  const float* band = p.ws_band + (int64_t)row * p.nband;

  if (p.nsp <= kFastChunks && p.nband <= kFastLabels) {
    // Few chunks and labels (the usual decoding step).  Every address below
    // depends on the launch parameters only, so all loads, the key length's
    // included, are in flight together: the row costs one memory round trip.
    // Slots past the row's position are masked afterwards.  Each thread
    // derives the row max and sum from all chunk scalars itself; the column
    // sums and the single-key weights are summed over the thread groups
    // (group g takes chunks and labels g, g + NG, ...).
    constexpr int UC = (kFastChunks + NG - 1) / NG, UL = (kFastLabels + NG - 1) / NG;
    const int t = row % p.Tq, bh = row / p.Tq;
    const int b = bh / p.H, h = bh - b * p.H;
    const int len_raw = p.cache_lens ? p.cache_lens[b] : p.L;
    float mlv[2 * kFastChunks], pov[UC], pmv[UC], blv[UL], wvv[UL];
    float w0 = 0.f;
#pragma unroll
    for (int c = 0; c < kFastChunks; ++c) {
      mlv[2 * c] = c < p.nsp ? ml[2 * c] : kNegInf;
      mlv[2 * c + 1] = c < p.nsp ? ml[2 * c + 1] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < UC; ++u) {
      const int c = grp + u * NG;
      pov[u] = c < p.nsp ? po[c * D + dim] : 0.f;
      pmv[u] = c < p.nsp ? ml[2 * c] : kNegInf;  // (indexing mlv by grp would spill)
    }
    if constexpr (VT) {
      // label slot x holds offset x + 1 - nband (labels -k+1 .. 0)
      const T* wvh = wv + h * p.wv_sh;
#pragma unroll
      for (int u = 0; u < UL; ++u) {
        const int x = grp + u * NG;
        blv[u] = x < p.nband ? band[x] : kNegInf;
        wvv[u] = x < p.nband ? (float)wvh[(x + 1 - p.nband + p.clip) * p.wv_sr + dim] : 0.f;
      }
      w0 = (float)wvh[dim];  // label -k
    }
    T* orow = reinterpret_cast<T*>(p.o) + b * p.o_sb + h * p.o_sh + t * p.o_st;
    const int i = min(max(len_raw, 0), p.L) - p.Tq + t;  // this query's position
    if (i < 0) {  // no visible key: zeros (whole workgroup)
      if (tid < D) orow[tid] = (T)0.f;
      return;
    }
    const int nchr = i / CH / p.cps + 1;  // splits holding keys 0..i
    float m = kNegInf;
#pragma unroll
    for (int c = 0; c < kFastChunks; ++c)
      if (c < nchr) m = fmaxf(m, mlv[2 * c]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int c = 0; c < kFastChunks; ++c)
      if (c < nchr) l = fmaf(mlv[2 * c + 1], fast_exp2(mlv[2 * c] - m), l);
#pragma unroll
    for (int u = 0; u < UC; ++u) {
      const int c = grp + u * NG;
      if (c < nchr) o = fmaf(pov[u], fast_exp2(pmv[u] - m), o);
    }
    float sbp = 0.f;  // this group's share of the single-key weights
    if constexpr (VT) {
#pragma unroll
      for (int u = 0; u < UL; ++u) {
        const int x = grp + u * NG;
        if (x < p.nband && x + 1 - p.nband >= -i) {  // the key at that offset exists
          const float w = fast_exp2(blv[u] - m);
          sbp += w;
          o = fmaf(w, wvv[u], o);
        }
      }
    }
    s_o[tid] = o;
    if (dim == 0) s_f[grp] = sbp;
    __syncthreads();
    if (tid < D) {
      float z = 0.f, sb = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        z += s_o[g * D + tid];
        sb += s_f[g];
      }
      if constexpr (VT) z = fmaf(fmaxf(l - sb, 0.f), w0, z);
      orow[tid] = (T)(z / l);
    }
    return;
  }

  const RowPos rp = row_pos(p, row);
  T* orow = reinterpret_cast<T*>(p.o) + rp.b * p.o_sb + rp.h * p.o_sh + rp.t * p.o_st;
  if (rp.i < 0) {  // no visible key: zeros (whole workgroup)
    if (tid < D) orow[tid] = (T)0.f;
    return;
  }
  const int nchr = rp.i / CH / p.cps + 1;  // splits holding keys 0..i
  const int lo = VT ? max(1 - p.nband, -rp.i) : 1;  // lowest offset with a single-key label
  const int cnt = 1 - lo;                             // single-key labels with a key
  float m = kNegInf;
  for (int c = tid; c < nchr; c += kDecThreads) m = fmaxf(m, ml[2 * c]);
  m = block_max(m, s_red, 0);
  // l = sum l_c 2^(m_c - m); column `dim` of O summed over this group's chunks
  float l = 0.f, o = 0.f;
  for (int c0 = 0; c0 < nchr; c0 += TILE) {
    const int nt = min(TILE, nchr - c0);
    for (int x = tid; x < nt; x += kDecThreads) {
      const float f = fast_exp2(ml[2 * (c0 + x)] - m);
      s_f[x] = f;
      l = fmaf(ml[2 * (c0 + x) + 1], f, l);
    }
    __syncthreads();
#pragma unroll 4
    for (int x = grp; x < nt; x += NG) o = fmaf(po[(int64_t)(c0 + x) * D + dim], s_f[x], o);
    __syncthreads();
  }
  l = block_sum(l, s_red, 1);
  if constexpr (MODE == kRelShaw && HAS_WV) {
    // labels -k+1 .. 0 hold one key each (when it exists); label -k (row 0)
    // holds every key at offset <= -k: what the row sum leaves
    const T* wvh = wv + rp.h * p.wv_sh;
    float sb = 0.f;
    for (int t0 = 0; t0 < cnt; t0 += TILE) {
      const int nt = min(TILE, cnt - t0);
      for (int x = tid; x < nt; x += kDecThreads) {
        const float w = fast_exp2(band[lo + t0 + x + p.nband - 1] - m);
        s_f[x] = w;
        sb += w;
      }
      __syncthreads();
#pragma unroll 4
      for (int x = grp; x < nt; x += NG)
        o = fmaf(s_f[x], (float)wvh[(int64_t)(lo + t0 + x + p.clip) * p.wv_sr + dim], o);
      __syncthreads();
    }
    sb = block_sum(sb, s_red, 2);
    if (grp == 0) o = fmaf(fmaxf(l - sb, 0.f), (float)wvh[dim], o);
  }
  s_o[tid] = o;
  __syncthreads();
  if (tid < D) {
    float z = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) z += s_o[g * D + tid];
    orow[tid] = (T)(z / l);
  }
}

template <int D, bool BF16, int MODE, bool HAS_WK, bool HAS_WV>
int launch_dec_t(const DecParams& p, hipStream_t s) {
  const int rows = p.B * p.H * p.Tq;
  if (p.direct) {
    hipLaunchKernelGGL((decode_kernel<D, BF16, MODE, HAS_WK, HAS_WV, true>), dim3(rows, 1),
                       dim3(kDecThreads), 0, s, p);
    return (int)hipGetLastError();
  }
  hipLaunchKernelGGL((decode_kernel<D, BF16, MODE, HAS_WK, HAS_WV, false>), dim3(rows, p.nsp),
                     dim3(kDecThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL((decode_combine_kernel<D, BF16, MODE, HAS_WV>), dim3(rows),
                     dim3(kDecThreads), 0, s, p);
  return (int)hipGetLastError();
}

template <int D, bool BF16>
int launch_dec_mode(RelMode mode, bool has_wk, bool has_wv, const DecParams& p, hipStream_t s) {
  if (mode == kRelT5) return launch_dec_t<D, BF16, kRelT5, false, false>(p, s);
  if (mode == kRelXL) return launch_dec_t<D, BF16, kRelXL, true, false>(p, s);
  if (mode == kRelShaw) {
    if (has_wk && has_wv) return launch_dec_t<D, BF16, kRelShaw, true, true>(p, s);
    if (has_wk) return launch_dec_t<D, BF16, kRelShaw, true, false>(p, s);
    return launch_dec_t<D, BF16, kRelShaw, false, true>(p, s);
  }
  return launch_dec_t<D, BF16, kRelNone, false, false>(p, s);
}

template <bool BF16>
int launch_dec_d(int d, RelMode mode, bool has_wk, bool has_wv, const DecParams& p,
                 hipStream_t s) {
  switch (d) {
    case 16: return launch_dec_mode<16, BF16>(mode, has_wk, has_wv, p, s);
    case 32: return launch_dec_mode<32, BF16>(mode, has_wk, has_wv, p, s);
    case 64: return launch_dec_mode<64, BF16>(mode, has_wk, has_wv, p, s);
    case 128: return launch_dec_mode<128, BF16>(mode, has_wk, has_wv, p, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_decode(bool bf16, int d, RelMode mode, bool has_wk, bool has_wv, const DecParams& p,
                  void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return bf16 ? launch_dec_d<true>(d, mode, has_wk, has_wv, p, s)
              : launch_dec_d<false>(d, mode, has_wk, has_wv, p, s);
}

}  // namespace relattn
