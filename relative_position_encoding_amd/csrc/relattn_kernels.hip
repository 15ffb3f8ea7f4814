// Fused forward of relation-aware self-attention for gfx950 (CDNA4).
//
// Method ("Self-Attention with Relative Position Representations", section
// 3.4, Eq. 3, Eq. 4 and the split of Eq. 5; T5 section of "Relative position
// embeddings"):
//   e_ij = scale * q_i.k_j + L[i, clip(j-i, c) + c],  L = scale * Q (w^K)^T
//   z_i  = (sum_j p_ij v_j + sum_r S[i, r] w^V_r) / sum_j p_ij
// with p_ij = exp(e_ij - m_i) and S[i, r] the sum of p_ij over the keys of
// label r.  T5 replaces L[i, .] by the per-head scalar bias of bucket
// beta(j - i) and drops the value term.
//
// One workgroup owns BR = 32 * NW query rows of one (batch, head); each wave
// owns 32 rows.  Both products run on 32x32 MFMA tiles laid out so that a
// lane owns ONE query row (column l & 31 of the tile) and half of the keys:
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16 / 32x32x2_f32), K from LDS, Q in
//                 registers for the whole kernel;
//   O^T += V^T P^T, P^T taken straight from the S^T accumulators, V^T read
//                 from a transposed LDS copy of the V tile.
// Because a lane owns a query, the online-softmax rescale of O, of the
// running sum and of the tail sums is a per-lane multiply; only the row max
// needs one cross-lane exchange per key tile.
//
// Relative key term: L is computed once per workgroup by one small MFMA
// product (BR x labels) and kept in LDS, one private row per query.  Inside
// the band |j - i| < c each logit gathers L[i, j-i+c]; outside the band the
// label is -c or +c for the whole tile, so two per-lane registers serve it.
//
// Relative value term: for |j - i| < c the bucket of label j-i+c holds a single
// key, so its weight is exp(e_ij - m_i): the kernel overwrites the gathered
// L[i, j-i+c] with the final logit e_ij (same LDS slot, same lane) and turns it
// into a weight in the epilogue once m_i is final.  The two tail buckets
// (labels -c and +c) are running sums rescaled like the row sum.  The
// epilogue then adds S W^V with one more MFMA product.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "relattn_internal.h"

namespace relattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Native vectors (HIP's uint4/uint2 are structs; copying those through memory
// keeps them out of registers).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// 2^x with the hardware exponential (about 1 ulp; results below 2^-126,
// which cannot change a softmax sum at fp32 precision, flush to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// Integer index functions.  The attention kernels and relattn_debug_indices
// both call these, so the dumped indices are the ones the kernels use.
// ---------------------------------------------------------------------------

// Table row of offset delta = j - i: clip(delta, c) + c (clip section).
__device__ __forceinline__ int clip_label(int delta, int c) {
  return min(max(delta, -c), c) + c;
}

// Bucket beta(delta) of the T5 section.
__device__ __forceinline__ int t5_bucket(int delta, const T5Buckets& t) {
  int base = 0;
  int a;
  if (t.bidir) {
    base = delta > 0 ? t.half : 0;
    a = delta < 0 ? -delta : delta;
  } else {
    a = delta < 0 ? -delta : 0;
  }
  if (a < t.exact) return base + a;
  int s = 0;
  for (int x = 0; x < t.nlog - 1; ++x) s += (a >= t.thr[x]) ? 1 : 0;
  return base + t.exact + s;
}

// Relative-logit rows in LDS hold the nr reachable labels between kRelPad
// copies of the first and of the last label on each side.
// With the padding, a group of 8 consecutive logits reads 8 consecutive
// entries from one clamped base index, whether the group lies in the band,
// in a tail or across an edge; no per-element clamp is needed.
constexpr int kRelPad = 16;

__host__ __device__ inline int label_row_stride_impl(int nr) {
  // even stride: consecutive query rows hit distinct LDS banks when the lanes
  // of a wave gather along a diagonal j - i
  return (nr + 2 * kRelPad + 1) & ~1;
}

// In-band logits are written back to a second row per query, indexed by
// label + 1 and clamped to [0, nr + 1]: entries 0 and nr + 1 take every logit
// outside the label window, and the tail labels take every logit of their
// tail; the epilogue reads only the in-band labels, so no per-element test
// is needed.  Even stride for the same bank argument as above.
__host__ __device__ inline int logit_row_stride_impl(int nr) { return (nr + 2 + 1) & ~1; }

// A row max may run ahead of the max used for the exponentials by this much
// (log2 units) before the running sums are rescaled: p <= 2^8 stays exact in
// fp32 sums and in bf16 operands, and most tiles then skip the rescale.
constexpr float kRescaleSlack = 8.f;

// Label rows of the value table staged in LDS, padded to whole MFMA steps.
__host__ __device__ inline int value_rows_padded(int nr) { return (nr + 15) & ~15; }

int label_row_stride(int nr) { return label_row_stride_impl(nr); }

// ---------------------------------------------------------------------------
// Tile geometry shared by the kernel and the host-side LDS sizing.
// ---------------------------------------------------------------------------
template <bool BF16, int D, int NW, int BC>
struct Geo {
  using T = std::conditional_t<BF16, __bf16, float>;
  static constexpr int BR = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int NKB = BC / 32;              // 32-key blocks per tile
  static constexpr int DVB = (D + 31) / 32;        // 32-wide d_v blocks
  static constexpr int KSTEP = BF16 ? 16 : 2;      // contraction per MFMA
  static constexpr int NKS = D / KSTEP;            // MFMAs over d
  static constexpr int KS = BF16 ? D + 8 : D + 4;  // K tile row stride
  // bf16: V stored transposed, Vt[d][key]; fp32: V[key][d].
  static constexpr int VS = BF16 ? BC + 8 : D + 4;
  static constexpr int K_ELEMS = BC * KS;
  static constexpr int V_ELEMS = BF16 ? D * VS : BC * VS;
  static constexpr size_t TILE_BYTES = (size_t)(K_ELEMS + V_ELEMS) * sizeof(T);
};

// Row of the K tile that feeds MFMA row m of a 32-key block.  The order is
// chosen so that accumulator register i of lane half h ends up holding key
// key_of_reg(i, h), which makes each lane's P values a ready MFMA operand for
// the P.V product (8 consecutive keys for bf16, 1 key for fp32).
template <bool BF16>
__device__ __forceinline__ int k_row_of_mfma_row(int m) {
  if constexpr (BF16) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);  // swap bits 2 and 3
  } else {
    return (m & ~7) | ((m & 3) << 1) | ((m >> 2) & 1);
  }
}

template <bool BF16>
__device__ __forceinline__ int key_of_reg(int i, int h) {
  if constexpr (BF16) {
    return 16 * (i >> 3) + 8 * h + (i & 7);
  } else {
    return 2 * i + h;
  }
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Workgroup id -> logical tile id.  Workgroups are dealt to the 8 XCDs round
// robin; this makes consecutive logical ids (tiles of the same batch and head,
// which share K and V) run on the same XCD and hence share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int per = G / 8, rem = G % 8, xcd = bid % 8, loc = bid / 8;
  return (xcd < rem) ? xcd * (per + 1) + loc
                     : rem * (per + 1) + (xcd - rem) * per + loc;
}

template <int D, int NW, int BC, bool BF16, int MODE, bool HAS_WK, bool HAS_WV>
__global__ __launch_bounds__(64 * NW) void fwd_kernel(const FwdParams p) {
  using G = Geo<BF16, D, NW, BC>;
  using T = typename G::T;
  using Op = std::conditional_t<BF16, bf16x8, float>;
  constexpr int BR = G::BR, NT = G::NT, NKB = G::NKB, DVB = G::DVB;
  constexpr int NKS = G::NKS, KS = G::KS, VS = G::VS;
  constexpr bool SHAW = (MODE == kRelShaw);
  constexpr bool T5 = (MODE == kRelT5);

  // ---- which tile
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / p.n_qtiles;
  int qt = lid - bh * p.n_qtiles;
  if (p.causal) qt = p.n_qtiles - 1 - qt;  // longest causal rows first
  const int b = bh / p.H, h = bh - b * p.H;
  const int i0 = qt * BR;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, hh = lane >> 5;
  const int qrow = wave * 32 + ql;
  const int qi = i0 + qrow;
  const bool q_ok = qi < p.n;
  const int wq0 = i0 + wave * 32;
  int kv_len = p.n;
  if (p.key_lens) kv_len = min(max(p.key_lens[b], 0), p.n);
  const int kv_end = p.causal ? min(kv_len, i0 + BR) : kv_len;
  const int kv_last = max(kv_len - 1, 0);
  const int c = p.clip;
  const int r_hi = p.r_lo + p.nr - 1;
  const int RS = label_row_stride_impl(p.nr);
  const int NRP = value_rows_padded(p.nr);

  // ---- LDS carve: K/V tile | L rows (Shaw) or bias-by-offset (T5) | w^V
  extern __shared__ __align__(16) unsigned char smem[];
  T* Ks = reinterpret_cast<T*>(smem);
  T* Vs = Ks + G::K_ELEMS;
  float* LE = reinterpret_cast<float*>(smem + G::TILE_BYTES);
  float* TB = LE;
  float* EB = LE + BR * RS;  // in-band logits (value term)
  const int ERS = logit_row_stride_impl(p.nr);
  T* WV = reinterpret_cast<T*>(EB + (HAS_WV ? BR * ERS : 0));
  float* myLE = LE + qrow * RS;
  float* myEB = EB + qrow * ERS;

  const T* qg = reinterpret_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const T* kg = reinterpret_cast<const T*>(p.k) + b * p.k_sb + h * p.k_sh;
  const T* vg = reinterpret_cast<const T*>(p.v) + b * p.v_sb + h * p.v_sh;
  T* og = reinterpret_cast<T*>(p.o) + b * p.o_sb + h * p.o_sh;

  // ---- Q as the B operand of S^T = K Q^T, resident for the whole kernel.
  // Rows past n load row n-1 (never stored); loads are unconditional so they
  // are all in flight together.
  Op qop[NKS];
  {
    const T* qrow_ptr = qg + (int64_t)min(qi, p.n - 1) * p.q_sn;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (BF16) {
        qop[ks] = *reinterpret_cast<const bf16x8*>(qrow_ptr + ks * 16 + 8 * hh);
      } else {
        qop[ks] = qrow_ptr[ks * 2 + hh];
      }
    }
  }

  // ---- K/V tile staging: global -> registers (prefetch) -> LDS.  Key rows
  // past the key length are clamped to the last visible row: their logits are
  // masked, so the values only need to be finite.
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  constexpr int K_CPR = D / EPC;
  constexpr int K_CHUNKS = BC * K_CPR;
  constexpr int K_PER_T = (K_CHUNKS + NT - 1) / NT;
  constexpr int V_UNITS = BF16 ? (BC / 4) * (D / 4) : K_CHUNKS;
  constexpr int V_PER_T = (V_UNITS + NT - 1) / NT;
  u32x4 kreg[K_PER_T];
  u32x2 vreg_b[BF16 ? V_PER_T : 1][4];
  u32x4 vreg_f[BF16 ? 1 : V_PER_T];

  auto load_tile = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < K_PER_T; ++u) {
      const int ch = min(tid + u * NT, K_CHUNKS - 1);
      const int row = ch / K_CPR, col = ch - row * K_CPR;
      const int j = min(j0 + row, kv_last);
      kreg[u] = *reinterpret_cast<const u32x4*>(kg + (int64_t)j * p.k_sn + col * EPC);
    }
    if constexpr (BF16) {
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u) {
        const int un = min(tid + u * NT, V_UNITS - 1);
        const int du = un % (D / 4), ku = un / (D / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = min(j0 + 4 * ku + r, kv_last);
          vreg_b[u][r] = *reinterpret_cast<const u32x2*>(vg + (int64_t)j * p.v_sn + 4 * du);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u) {
        const int ch = min(tid + u * NT, K_CHUNKS - 1);
        const int row = ch / K_CPR, col = ch - row * K_CPR;
        const int j = min(j0 + row, kv_last);
        vreg_f[u] = *reinterpret_cast<const u32x4*>(vg + (int64_t)j * p.v_sn + col * EPC);
      }
    }
  };

  auto store_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < K_PER_T; ++u) {
      const int ch = tid + u * NT;
      const int row = ch / K_CPR, col = ch - row * K_CPR;
      if (K_CHUNKS % NT == 0 || ch < K_CHUNKS)
        *reinterpret_cast<u32x4*>(Ks + row * KS + col * EPC) = kreg[u];
    }
    if constexpr (BF16) {
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u) {
        const int un = tid + u * NT;
        const int du = un % (D / 4), ku = un / (D / 4);
        const u32x2* r = vreg_b[u];
        // 4x4 transpose of 16-bit values: column e of the 4 rows -> Vt row 4du+e
        u32x2 col[4];
        col[0].x = (r[0].x & 0xffffu) | (r[1].x << 16);
        col[0].y = (r[2].x & 0xffffu) | (r[3].x << 16);
        col[1].x = (r[0].x >> 16) | (r[1].x & 0xffff0000u);
        col[1].y = (r[2].x >> 16) | (r[3].x & 0xffff0000u);
        col[2].x = (r[0].y & 0xffffu) | (r[1].y << 16);
        col[2].y = (r[2].y & 0xffffu) | (r[3].y << 16);
        col[3].x = (r[0].y >> 16) | (r[1].y & 0xffff0000u);
        col[3].y = (r[2].y >> 16) | (r[3].y & 0xffff0000u);
        if (V_UNITS % NT == 0 || un < V_UNITS) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            *reinterpret_cast<u32x2*>(Vs + (4 * du + e) * VS + 4 * ku) = col[e];
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u) {
        const int ch = tid + u * NT;
        const int row = ch / K_CPR, col = ch - row * K_CPR;
        if (K_CHUNKS % NT == 0 || ch < K_CHUNKS)
          *reinterpret_cast<u32x4*>(Vs + row * VS + col * EPC) = vreg_f[u];
      }
    }
  };

  const int ntiles = (kv_end + BC - 1) / BC;
  if (ntiles > 0) load_tile(0);  // in flight while the tables are prepared

  // ---- relative logits in LDS.  Shaw: row qrow holds scale*log2e*q.w^K_r for
  // the reachable label rows r_lo..r_hi at entries kRelPad + (r - r_lo).  T5:
  // one shared vector holds log2e*bias[beta(delta), h] for delta in
  // [-dist, dist] at entries kRelPad + dist + delta.  Both are padded.
  if constexpr (SHAW) {
    if constexpr (HAS_WK) {
      const T* wkh = reinterpret_cast<const T*>(p.wk) + h * p.wk_sh;
      const int nlb = (p.nr + 31) / 32;
      for (int lb = 0; lb < nlb; ++lb) {
        // MFMA row m = ql <-> label row r_lo + lb*32 + ql (clamped; rows past
        // the window produce values that are never stored)
        const T* wrow = wkh + (int64_t)min(p.r_lo + lb * 32 + ql, r_hi) * p.wk_sr;
        Op a[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if constexpr (BF16) {
            a[ks] = *reinterpret_cast<const bf16x8*>(wrow + ks * 16 + 8 * hh);
          } else {
            a[ks] = wrow[ks * 2 + hh];
          }
        }
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) acc = mfma(a[ks], qop[ks], acc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int idx = lb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (idx < p.nr) myLE[kRelPad + idx] = acc[i] * p.scale_log2;
        }
      }
    } else {
      for (int idx = hh; idx < p.nr + 2 * kRelPad; idx += 2) myLE[idx] = 0.f;
    }
    if constexpr (HAS_WV) {
      // value table rows r_lo .. r_hi (zero past nr): bf16 transposed to
      // WV[d][label] so a lane reads 8 labels of one d with one 16-byte load;
      // fp32 kept as WV[label][d].
      const T* wvh = reinterpret_cast<const T*>(p.wv) + h * p.wv_sh;
      constexpr int CPR = D / EPC;
      const int nch = NRP * CPR;
      for (int u = tid; u < nch; u += NT) {
        const int idx = u / CPR, ch = u - idx * CPR;
        const T* src = wvh + (int64_t)(p.r_lo + min(idx, p.nr - 1)) * p.wv_sr + ch * EPC;
        u32x4 val = *reinterpret_cast<const u32x4*>(src);
        if (idx >= p.nr) val = u32x4{0u, 0u, 0u, 0u};
        if constexpr (BF16) {
          const int WS = NRP + 8;
          const unsigned w32[4] = {val.x, val.y, val.z, val.w};
          unsigned short* dst = reinterpret_cast<unsigned short*>(WV);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            dst[(ch * 8 + e) * WS + idx] = (unsigned short)(w32[e >> 1] >> (16 * (e & 1)));
        } else {
          *reinterpret_cast<u32x4*>(WV + idx * (D + 4) + ch * 4) = val;
        }
      }
    }
  }
  if constexpr (T5) {
    const int nb = 2 * p.t5_dist + 1 + 2 * kRelPad;
    for (int x = tid; x < nb; x += NT) {
      const int delta = min(max(x - kRelPad - p.t5_dist, -p.t5_dist), p.t5_dist);
      TB[x] = kLog2e * p.t5_bias[t5_bucket(delta, p.t5) * p.tb_sb + h * p.tb_sh];
    }
  }
  __syncthreads();
  if constexpr (SHAW && HAS_WK) {
    // replicate the first / last label into the padding of this row
    const float edge = myLE[hh ? kRelPad + p.nr - 1 : kRelPad];
    float* pad = myLE + (hh ? kRelPad + p.nr : 0);
#pragma unroll
    for (int x = 0; x < kRelPad; ++x) pad[x] = edge;
  }
  __syncthreads();

  // window of offsets delta = j - i covered by the relative row, and the
  // relative logit of the two ends (used for tiles entirely outside the band)
  const int dlo = T5 ? -p.t5_dist : p.r_lo - c;           // delta of entry kRelPad
  const int nwin = T5 ? 2 * p.t5_dist + 1 : p.nr;
  const float* relrow = T5 ? TB : myLE;
  float Llo = 0.f, Lhi = 0.f;
  if constexpr (SHAW || T5) {
    Llo = relrow[kRelPad];
    Lhi = relrow[kRelPad + nwin - 1];
  }
  const int band = T5 ? p.t5_dist : c;  // |j - i| >= band: one end value for the tile

  // ---- running state (per lane: one query, half of each tile's keys)
  f32x16 oacc[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) oacc[mb] = f32x16{};
  float m_run = kNegInf;
  float l_part = 0.f, thi = 0.f;
  const int hi_from = max(c, 1 - c);  // offsets >= hi_from fall in the +c bucket
  constexpr int KSTR = BF16 ? 1 : 2;  // key step between consecutive registers
  constexpr int SPAN = 7 * KSTR + 1;  // keys spanned by a group of 8 registers
  const int hoff = BF16 ? 8 * hh : hh;  // key offset of this lane half

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * BC;
    __syncthreads();  // every wave is done with the previous tile
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(j0 + BC);

    if (wq0 >= p.n) continue;                  // no live query in this wave
    if (p.causal && j0 > wq0 + 31) continue;   // tile entirely in the future

    // S^T block kb: rows = keys j0 + 32kb + .., columns = this wave's queries
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      // all K fragments of the block first, then the MFMA chain
      const int krow = 32 * kb + k_row_of_mfma_row<BF16>(ql);
      Op a[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if constexpr (BF16) {
          a[ks] = *reinterpret_cast<const bf16x8*>(Ks + krow * KS + ks * 16 + 8 * hh);
        } else {
          a[ks] = Ks[krow * KS + ks * 2 + hh];
        }
      }
      s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) s[kb] = mfma(a[ks], qop[ks], s[kb]);
    }

    // Register (kb, 8g + e) holds key j0 + hoff + 32kb + 16g + KSTR*e, i.e.
    // offset delta = kofs + 32kb + 16g + KSTR*e from this lane's query.
    const int kofs = j0 + hoff - qi;
    const bool need_mask = (j0 + BC > kv_len) || (p.causal && j0 + BC - 1 > wq0);
    // visible iff its key offset within the lane's keys is <= lim
    const int lim = min(kv_len - 1 - j0 - hoff, p.causal ? -kofs : 0x3fffffff);
    const int dmin = j0 - (wq0 + 31), dmax = j0 + BC - 1 - wq0;
    const bool all_lo = dmax <= -band, all_hi = dmin >= band;  // wave-uniform
    const bool off_band = (SHAW || T5) && (all_lo || all_hi);
    float tmax = kNegInf;
    if (!(SHAW || T5) || off_band) {
      // no relative term, or one end value for the whole tile
      const float rel = (SHAW || T5) ? (all_lo ? Llo : Lhi) : 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ko = 32 * kb + 16 * (i >> 3) + KSTR * (i & 7);
          float x = fmaf(s[kb][i], p.scale_log2, rel);
          if (need_mask) x = (ko <= lim) ? x : kNegInf;
          s[kb][i] = x;
          tmax = fmaxf(tmax, x);
        }
    } else {
      // band: gather every relative logit of the tile first (8 consecutive
      // entries per group from one clamped base, see kRelPad), then combine
      float rv[NKB][16];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int d0 = kofs + 32 * kb + 16 * g;  // offset of the group's first key
          const int bidx = min(max(d0 - dlo + kRelPad, 0), nwin + 2 * kRelPad - SPAN);
          const float* grp = relrow + bidx;
#pragma unroll
          for (int e = 0; e < 8; ++e) rv[kb][8 * g + e] = grp[KSTR * e];
        }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ko = 32 * kb + 16 * (i >> 3) + KSTR * (i & 7);
          float x = fmaf(s[kb][i], p.scale_log2, rv[kb][i]);
          if (need_mask) x = (ko <= lim) ? x : kNegInf;
          rv[kb][i] = x;  // unmasked logits of visible keys are kept for write-back
          s[kb][i] = x;
          tmax = fmaxf(tmax, x);
        }
      if constexpr (SHAW && HAS_WV) {
        // logits to their label slot of the write-back row (see
        // logit_row_stride_impl); masked keys are harmless there because the
        // epilogue re-checks visibility
        const int wbase = kofs + c - p.r_lo + 1;  // entry of key offset 0
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ko = 32 * kb + 16 * (i >> 3) + KSTR * (i & 7);
            myEB[min(max(wbase + ko, 0), p.nr + 1)] = rv[kb][i];
          }
      }
    }

    // online softmax: one cross-lane max per tile, everything else per lane
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const bool grow = tmax > m_run + kRescaleSlack;  // -inf + slack is -inf
    if (__any(grow)) {  // wave-uniform
      const float m_next = grow ? tmax : m_run;
      const float alpha = fast_exp2(m_run - m_next);  // 0 when m_run is -inf
      m_run = m_next;
      l_part *= alpha;
      if constexpr (SHAW && HAS_WV) thi *= alpha;
#pragma unroll
      for (int mb = 0; mb < DVB; ++mb) oacc[mb] *= alpha;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;

    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(s[kb][i] - m_use);
        s[kb][i] = pv;
        psum += pv;
      }
    }
    l_part += psum;
    if constexpr (SHAW && HAS_WV) {
      // +c bucket (keys at offset >= c); empty under the causal mask
      if (!p.causal && !all_lo) {
        if (all_hi) {
          thi += psum;
        } else {
          const int hi_ko = hi_from - kofs;  // first key offset in the +c bucket
          float phi = 0.f;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int ko = 32 * kb + 16 * (i >> 3) + KSTR * (i & 7);
              phi += (ko >= hi_ko) ? s[kb][i] : 0.f;
            }
          thi += phi;
        }
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if constexpr (BF16) {
        bf16x8 va[2][DVB];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) {
            const int dv = min(32 * mb + ql, D - 1);  // rows past D are never stored
            va[t2][mb] =
                *reinterpret_cast<const bf16x8*>(Vs + dv * VS + 32 * kb + 16 * t2 + 8 * hh);
          }
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[kb][8 * t2 + e];
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) oacc[mb] = mfma(va[t2][mb], pb, oacc[mb]);
        }
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) {
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) {
            const int dv = min(32 * mb + ql, D - 1);
            const float a = Vs[(32 * kb + 2 * s2 + hh) * VS + dv];
            oacc[mb] = mfma(a, s[kb][s2], oacc[mb]);
          }
        }
      }
    }
  }
  __syncthreads();  // logits written to LE by both lane halves are visible

  // ---- epilogue
  const float l = l_part + __shfl_xor(l_part, 32);
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  if constexpr (SHAW && HAS_WV) {
    const float thi_all = thi + __shfl_xor(thi, 32);
    const float m_fin = (m_run == kNegInf) ? 0.f : m_run;
    // weight of an in-band label row (r_lo + idx): the single key it holds
    auto interior_weight = [&](int idx) __attribute__((always_inline)) -> float {
      const int r = p.r_lo + idx;
      const int j = qi + r - c;
      const bool ok = idx < p.nr && q_ok && r > 0 && r < 2 * c && j >= 0 && j < kv_len &&
                      (!p.causal || j <= qi);
      const float e = myEB[1 + min(idx, p.nr - 1)];
      return ok ? fast_exp2(e - m_fin) : 0.f;
    };
    // the -c bucket holds what the row sum leaves after the band and the +c bucket
    float isum = 0.f;
    for (int idx = hh; idx < p.nr; idx += 2) isum += interior_weight(idx);
    isum += __shfl_xor(isum, 32);
    const float tlo_all = fmaxf(l - isum - thi_all, 0.f);
    auto bucket_weight = [&](int idx) __attribute__((always_inline)) -> float {
      const int r = p.r_lo + idx;
      const float w = (r == 0 ? tlo_all : 0.f) + (r == 2 * c ? thi_all : 0.f);
      return (idx < p.nr && q_ok) ? w + interior_weight(idx) : 0.f;
    };
    constexpr int LSTEP = BF16 ? 16 : 2;
    const int nls = NRP / LSTEP;
    for (int ls = 0; ls < nls; ++ls) {
      if constexpr (BF16) {
        bf16x8 bw;
#pragma unroll
        for (int e = 0; e < 8; ++e) bw[e] = (__bf16)bucket_weight(ls * 16 + 8 * hh + e);
        const int WS = NRP + 8;
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb) {
          const int dv = min(32 * mb + ql, D - 1);
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(WV + dv * WS + ls * 16 + 8 * hh);
          oacc[mb] = mfma(a, bw, oacc[mb]);
        }
      } else {
        const int idx = ls * 2 + hh;
        const float bw = bucket_weight(idx);
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb) {
          const int dv = min(32 * mb + ql, D - 1);
          oacc[mb] = mfma(WV[idx * (D + 4) + dv], bw, oacc[mb]);
        }
      }
    }
  }

  if (q_ok) {
    T* orow = og + (int64_t)qi * p.o_sn;
#pragma unroll
    for (int mb = 0; mb < DVB; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dv0 = 32 * mb + 8 * g + 4 * hh;
        if (dv0 < D) {
          if constexpr (BF16) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[mb][4 * g + e] * inv_l);
            *reinterpret_cast<bf16x4*>(orow + dv0) = o4;
          } else {
            f32x4 o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = oacc[mb][4 * g + e] * inv_l;
            *reinterpret_cast<f32x4*>(orow + dv0) = o4;
          }
        }
      }
    }
  }
}

__global__ void debug_indices_kernel(int n, int clip, T5Buckets t5, int use_t5,
                                     int32_t* out) {
  const int x = blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= 2 * n - 1) return;
  const int delta = x - (n - 1);
  out[x] = use_t5 ? t5_bucket(delta, t5) : clip_label(delta, clip);
}

// ---------------------------------------------------------------------------
// host side: LDS sizing and dispatch over the compiled variants
// ---------------------------------------------------------------------------

template <bool BF16, int D, int NW, int BC>
static size_t lds_bytes_t(RelMode mode, bool has_wv, int nr, int t5_dist) {
  using G = Geo<BF16, D, NW, BC>;
  size_t extra = 0;
  if (mode == kRelShaw) {
    extra = (size_t)G::BR * label_row_stride_impl(nr) * sizeof(float);
    if (has_wv) {
      extra += (size_t)G::BR * logit_row_stride_impl(nr) * sizeof(float);
      const size_t nrp = value_rows_padded(nr);
      extra += BF16 ? (size_t)D * (nrp + 8) * 2 : nrp * (D + 4) * 4;
    }
  }
  if (mode == kRelT5) extra = (size_t)(2 * t5_dist + 1 + 2 * kRelPad) * sizeof(float);
  return G::TILE_BYTES + extra;
}

constexpr int kBlockKeys = 64;  // BC for bf16
constexpr int kBlockKeysF32 = 32;

size_t lds_bytes(bool bf16, int d, const LaunchCfg& cfg, RelMode mode, bool has_wv,
                 int nr, int t5_dist) {
#define RELATTN_LDS(BF, DD, NWW, BCC) \
  if (bf16 == BF && d == DD && cfg.waves == NWW && cfg.kblock == BCC) \
    return lds_bytes_t<BF, DD, NWW, BCC>(mode, has_wv, nr, t5_dist);
#define RELATTN_LDS_D(BF, NWW, BCC) \
  RELATTN_LDS(BF, 16, NWW, BCC) RELATTN_LDS(BF, 32, NWW, BCC) \
  RELATTN_LDS(BF, 64, NWW, BCC) RELATTN_LDS(BF, 128, NWW, BCC)
  RELATTN_LDS_D(true, 1, kBlockKeys)
  RELATTN_LDS_D(true, 2, kBlockKeys)
  RELATTN_LDS_D(true, 4, kBlockKeys)
  RELATTN_LDS_D(false, 1, kBlockKeysF32)
  RELATTN_LDS_D(false, 2, kBlockKeysF32)
#undef RELATTN_LDS_D
#undef RELATTN_LDS
  return 0;
}

template <int D, int NW, int BC, bool BF16, int MODE, bool HAS_WK, bool HAS_WV>
static int launch_t(const FwdParams& p, void* stream) {
  auto kern = fwd_kernel<D, NW, BC, BF16, MODE, HAS_WK, HAS_WV>;
  const size_t lds = lds_bytes_t<BF16, D, NW, BC>((RelMode)MODE, HAS_WV, p.nr, p.t5_dist);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return (int)e;
  }
  const long long grid = (long long)p.B * p.H * p.n_qtiles;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * NW), lds,
                     reinterpret_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

template <int D, int NW, int BC, bool BF16>
static int launch_mode(RelMode mode, bool has_wk, bool has_wv, const FwdParams& p,
                       void* stream) {
  if (mode == kRelT5) return launch_t<D, NW, BC, BF16, kRelT5, false, false>(p, stream);
  if (mode == kRelShaw) {
    if (has_wk && has_wv) return launch_t<D, NW, BC, BF16, kRelShaw, true, true>(p, stream);
    if (has_wk) return launch_t<D, NW, BC, BF16, kRelShaw, true, false>(p, stream);
    if (has_wv) return launch_t<D, NW, BC, BF16, kRelShaw, false, true>(p, stream);
  }
  return launch_t<D, NW, BC, BF16, kRelNone, false, false>(p, stream);
}

template <int NW, int BC, bool BF16>
static int launch_d(int d, RelMode mode, bool has_wk, bool has_wv, const FwdParams& p,
                    void* stream) {
  switch (d) {
    case 16: return launch_mode<16, NW, BC, BF16>(mode, has_wk, has_wv, p, stream);
    case 32: return launch_mode<32, NW, BC, BF16>(mode, has_wk, has_wv, p, stream);
    case 64: return launch_mode<64, NW, BC, BF16>(mode, has_wk, has_wv, p, stream);
    case 128: return launch_mode<128, NW, BC, BF16>(mode, has_wk, has_wv, p, stream);
  }
  return (int)hipErrorInvalidValue;
}

int launch_fwd(bool bf16, int d, const LaunchCfg& cfg, RelMode mode, bool has_wk,
               bool has_wv, const FwdParams& p, void* stream) {
  if (bf16) {
    if (cfg.kblock != kBlockKeys) return (int)hipErrorInvalidValue;
    if (cfg.waves == 1) return launch_d<1, kBlockKeys, true>(d, mode, has_wk, has_wv, p, stream);
    if (cfg.waves == 2) return launch_d<2, kBlockKeys, true>(d, mode, has_wk, has_wv, p, stream);
    if (cfg.waves == 4) return launch_d<4, kBlockKeys, true>(d, mode, has_wk, has_wv, p, stream);
  } else {
    if (cfg.kblock != kBlockKeysF32) return (int)hipErrorInvalidValue;
    if (cfg.waves == 1) return launch_d<1, kBlockKeysF32, false>(d, mode, has_wk, has_wv, p, stream);
    if (cfg.waves == 2) return launch_d<2, kBlockKeysF32, false>(d, mode, has_wk, has_wv, p, stream);
  }
  return (int)hipErrorInvalidValue;
}

int launch_debug_indices(int n, int clip, const T5Buckets* t5, int32_t* out, void* stream) {
  const int total = 2 * n - 1;
  const int threads = 256;
  const int blocks = (total + threads - 1) / threads;
  T5Buckets tb = {};
  if (t5) tb = *t5;
  hipLaunchKernelGGL(debug_indices_kernel, dim3(blocks), dim3(threads), 0,
                     reinterpret_cast<hipStream_t>(stream), n, clip, tb, t5 ? 1 : 0, out);
  return (int)hipGetLastError();
}

}  // namespace relattn
