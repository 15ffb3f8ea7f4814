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

constexpr float kLog2e = 1.4426950408889634f;
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

__host__ __device__ inline int label_row_stride_impl(int nr) {
  // Even stride: consecutive query rows then hit distinct LDS banks when the
  // lanes of a wave gather along a diagonal j - i.
  return (nr & 1) ? nr + 1 : nr;
}

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
  constexpr int KSTEP = G::KSTEP, NKS = G::NKS, KS = G::KS, VS = G::VS;
  constexpr bool SHAW = (MODE == kRelShaw);
  constexpr bool T5 = (MODE == kRelT5);

  extern __shared__ __align__(16) unsigned char smem[];
  T* Ks = reinterpret_cast<T*>(smem);
  T* Vs = Ks + G::K_ELEMS;
  float* LE = reinterpret_cast<float*>(smem + G::TILE_BYTES);  // Shaw: L rows
  float* TB = LE;                                              // T5: bias by offset

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
  const int c = p.clip;
  const int r_hi = p.r_lo + p.nr - 1;

  const T* qg = reinterpret_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const T* kg = reinterpret_cast<const T*>(p.k) + b * p.k_sb + h * p.k_sh;
  const T* vg = reinterpret_cast<const T*>(p.v) + b * p.v_sb + h * p.v_sh;
  T* og = reinterpret_cast<T*>(p.o) + b * p.o_sb + h * p.o_sh;

  // ---- Q as the B operand of S^T = K Q^T, resident for the whole kernel
  Op qop[NKS];
  {
    const T* qrow_ptr = qg + (int64_t)qi * p.q_sn;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (BF16) {
        qop[ks] = q_ok ? *reinterpret_cast<const bf16x8*>(qrow_ptr + ks * 16 + 8 * hh)
                       : bf16x8{};
      } else {
        qop[ks] = q_ok ? qrow_ptr[ks * 2 + hh] : 0.f;
      }
    }
  }

  // ---- relative key logits L (Shaw) or bias-by-offset vector (T5), in LDS
  const int RS = label_row_stride_impl(p.nr);
  float* myLE = LE + qrow * RS;
  if constexpr (SHAW) {
    if constexpr (HAS_WK) {
      const T* wkh = reinterpret_cast<const T*>(p.wk) + h * p.wk_sh;
      const int nlb = (p.nr + 31) / 32;
      for (int lb = 0; lb < nlb; ++lb) {
        const int arow = lb * 32 + ql;  // MFMA row m = ql <-> label row r_lo + arow
        const bool a_ok = arow < p.nr;
        const T* wrow = wkh + (int64_t)(p.r_lo + (a_ok ? arow : 0)) * p.wk_sr;
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          Op a;
          if constexpr (BF16) {
            a = a_ok ? *reinterpret_cast<const bf16x8*>(wrow + ks * 16 + 8 * hh) : bf16x8{};
          } else {
            a = a_ok ? wrow[ks * 2 + hh] : 0.f;
          }
          acc = mfma(a, qop[ks], acc);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int idx = lb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (idx < p.nr) myLE[idx] = acc[i] * p.scale_log2;
        }
      }
    } else {
      for (int idx = hh; idx < p.nr; idx += 2) myLE[idx] = 0.f;
    }
  }
  if constexpr (T5) {
    const int nb = 2 * p.t5_dist + 1;
    for (int x = tid; x < nb; x += NT) {
      const int bucket = t5_bucket(x - p.t5_dist, p.t5);
      TB[x] = kLog2e * p.t5_bias[bucket * p.tb_sb + h * p.tb_sh];
    }
  }
  __syncthreads();
  float Llo = 0.f, Lhi = 0.f;  // L at labels -c and +c (clamped into the window)
  if constexpr (SHAW && HAS_WK) {
    Llo = myLE[min(max(0, p.r_lo), r_hi) - p.r_lo];
    Lhi = myLE[min(max(2 * c, p.r_lo), r_hi) - p.r_lo];
  }

  // ---- K/V tile staging: global -> registers (prefetch) -> LDS
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  constexpr int K_CPR = D / EPC;
  constexpr int K_CHUNKS = BC * K_CPR;
  constexpr int K_PER_T = (K_CHUNKS + NT - 1) / NT;
  constexpr int V_UNITS = BF16 ? (BC / 4) * (D / 4) : K_CHUNKS;
  constexpr int V_PER_T = (V_UNITS + NT - 1) / NT;
  uint4 kreg[K_PER_T];
  uint2 vreg_b[BF16 ? V_PER_T : 1][4];
  uint4 vreg_f[BF16 ? 1 : V_PER_T];

  auto load_tile = [&](int j0) {
#pragma unroll
    for (int u = 0; u < K_PER_T; ++u) {
      const int ch = tid + u * NT;
      const int row = ch / K_CPR, col = ch - row * K_CPR;
      const int j = j0 + row;
      uint4 val = {0u, 0u, 0u, 0u};
      if (ch < K_CHUNKS && j < kv_len)
        val = *reinterpret_cast<const uint4*>(kg + (int64_t)j * p.k_sn + col * EPC);
      kreg[u] = val;
    }
    if constexpr (BF16) {
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u) {
        const int un = tid + u * NT;
        const int du = un % (D / 4), ku = un / (D / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + 4 * ku + r;
          uint2 val = {0u, 0u};
          if (un < V_UNITS && j < kv_len)
            val = *reinterpret_cast<const uint2*>(vg + (int64_t)j * p.v_sn + 4 * du);
          vreg_b[u][r] = val;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u) {
        const int ch = tid + u * NT;
        const int row = ch / K_CPR, col = ch - row * K_CPR;
        const int j = j0 + row;
        uint4 val = {0u, 0u, 0u, 0u};
        if (ch < K_CHUNKS && j < kv_len)
          val = *reinterpret_cast<const uint4*>(vg + (int64_t)j * p.v_sn + col * EPC);
        vreg_f[u] = val;
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < K_PER_T; ++u) {
      const int ch = tid + u * NT;
      const int row = ch / K_CPR, col = ch - row * K_CPR;
      if (ch < K_CHUNKS) *reinterpret_cast<uint4*>(Ks + row * KS + col * EPC) = kreg[u];
    }
    if constexpr (BF16) {
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u) {
        const int un = tid + u * NT;
        if (un >= V_UNITS) continue;
        const int du = un % (D / 4), ku = un / (D / 4);
        const uint2* r = vreg_b[u];
        // 4x4 transpose of 16-bit values: column e of the 4 rows -> Vt row 4du+e
        uint2 col[4];
        col[0].x = (r[0].x & 0xffffu) | (r[1].x << 16);
        col[0].y = (r[2].x & 0xffffu) | (r[3].x << 16);
        col[1].x = (r[0].x >> 16) | (r[1].x & 0xffff0000u);
        col[1].y = (r[2].x >> 16) | (r[3].x & 0xffff0000u);
        col[2].x = (r[0].y & 0xffffu) | (r[1].y << 16);
        col[2].y = (r[2].y & 0xffffu) | (r[3].y << 16);
        col[3].x = (r[0].y >> 16) | (r[1].y & 0xffff0000u);
        col[3].y = (r[2].y >> 16) | (r[3].y & 0xffff0000u);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<uint2*>(Vs + (4 * du + e) * VS + 4 * ku) = col[e];
      }
    } else {
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u) {
        const int ch = tid + u * NT;
        const int row = ch / K_CPR, col = ch - row * K_CPR;
        if (ch < K_CHUNKS) *reinterpret_cast<uint4*>(Vs + row * VS + col * EPC) = vreg_f[u];
      }
    }
  };

  // ---- running state (per lane: one query, half of each tile's keys)
  f32x16 oacc[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) oacc[mb] = f32x16{};
  float m_run = kNegInf;
  float l_part = 0.f, tlo = 0.f, thi = 0.f;
  const int hi_from = max(c, 1 - c);  // offsets >= hi_from fall in the +c bucket

  const int ntiles = (kv_end + BC - 1) / BC;
  if (ntiles > 0) load_tile(0);
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
      s[kb] = f32x16{};
      const int krow = 32 * kb + k_row_of_mfma_row<BF16>(ql);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        Op a;
        if constexpr (BF16) {
          a = *reinterpret_cast<const bf16x8*>(Ks + krow * KS + ks * 16 + 8 * hh);
        } else {
          a = Ks[krow * KS + ks * 2 + hh];
        }
        s[kb] = mfma(a, qop[ks], s[kb]);
      }
    }

    // logits in log2 units, relative term, masks
    const bool need_mask = (j0 + BC > kv_len) || (p.causal && j0 + BC - 1 > wq0);
    const int dmin = j0 - (wq0 + 31), dmax = j0 + BC - 1 - wq0;
    const bool all_lo = dmax <= -c, all_hi = dmin >= c;
    const bool tail_lo = all_lo, tail_hi = dmin >= hi_from;  // whole tile in one tail
    float tmax = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = j0 + 32 * kb + key_of_reg<BF16>(i, hh);
        const int delta = j - qi;
        float x = s[kb][i] * p.scale_log2;
        bool vis = true;
        if (need_mask) vis = (j < kv_len) && (!p.causal || j <= qi);
        if constexpr (SHAW) {
          if (all_lo) {
            x += Llo;
          } else if (all_hi) {
            x += Lhi;
          } else {
            const int slot = min(max(clip_label(delta, c), p.r_lo), r_hi) - p.r_lo;
            if constexpr (HAS_WK) x += myLE[slot];
            if constexpr (HAS_WV) {
              if (vis && q_ok && delta > -c && delta < c) myLE[slot] = x;
            }
          }
        }
        if constexpr (T5) {
          x += TB[min(max(delta, -p.t5_dist), p.t5_dist) + p.t5_dist];
        }
        x = vis ? x : kNegInf;
        s[kb][i] = x;
        tmax = fmaxf(tmax, x);
      }
    }

    // online softmax: one cross-lane max per tile, everything else per lane
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    l_part *= alpha;
    tlo *= alpha;
    thi *= alpha;
#pragma unroll
    for (int mb = 0; mb < DVB; ++mb) oacc[mb] *= alpha;

    float psum = 0.f, plo = 0.f, phi = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = exp2f(s[kb][i] - m_use);
        s[kb][i] = pv;
        psum += pv;
        if constexpr (SHAW && HAS_WV) {
          if (!tail_lo && !tail_hi) {
            const int delta = j0 + 32 * kb + key_of_reg<BF16>(i, hh) - qi;
            if (delta <= -c) plo += pv;
            else if (delta >= hi_from) phi += pv;
          }
        }
      }
    }
    l_part += psum;
    if constexpr (SHAW && HAS_WV) {
      if (tail_lo) plo = psum;
      else if (tail_hi) phi = psum;
      tlo += plo;
      thi += phi;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if constexpr (BF16) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[kb][8 * t2 + e];
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) {
            const int dv = 32 * mb + ql;
            const bf16x8 a = (dv < D)
                ? *reinterpret_cast<const bf16x8*>(Vs + dv * VS + 32 * kb + 16 * t2 + 8 * hh)
                : bf16x8{};
            oacc[mb] = mfma(a, pb, oacc[mb]);
          }
        }
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) {
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) {
            const int dv = 32 * mb + ql;
            const float a = (dv < D) ? Vs[(32 * kb + 2 * s2 + hh) * VS + dv] : 0.f;
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
    const float tlo_all = tlo + __shfl_xor(tlo, 32);
    const float thi_all = thi + __shfl_xor(thi, 32);
    const float m_fin = (m_run == kNegInf) ? 0.f : m_run;
    const T* wvh = reinterpret_cast<const T*>(p.wv) + h * p.wv_sh;
    // weight of label row (r_lo + idx) for this lane's query
    auto bucket_weight = [&](int idx) -> float {
      if (idx >= p.nr || !q_ok) return 0.f;
      const int r = p.r_lo + idx;
      float w = 0.f;
      if (r == 0) w += tlo_all;
      if (r == 2 * c) w += thi_all;
      if (r > 0 && r < 2 * c) {
        const int j = qi + r - c;
        const bool vis = j >= 0 && j < kv_len && (!p.causal || j <= qi);
        if (vis) w = exp2f(myLE[idx] - m_fin);
      }
      return w;
    };
    constexpr int LSTEP = BF16 ? 16 : 2;
    const int nls = (p.nr + LSTEP - 1) / LSTEP;
    for (int ls = 0; ls < nls; ++ls) {
      if constexpr (BF16) {
        bf16x8 bw;
#pragma unroll
        for (int e = 0; e < 8; ++e) bw[e] = (__bf16)bucket_weight(ls * 16 + 8 * hh + e);
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb) {
          const int dv = 32 * mb + ql;
          bf16x8 a;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int idx = ls * 16 + 8 * hh + e;
            a[e] = (idx < p.nr && dv < D) ? wvh[(int64_t)(p.r_lo + idx) * p.wv_sr + dv]
                                          : (__bf16)0.f;
          }
          oacc[mb] = mfma(a, bw, oacc[mb]);
        }
      } else {
        const int idx = ls * 2 + hh;
        const float bw = bucket_weight(idx);
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb) {
          const int dv = 32 * mb + ql;
          const float a = (idx < p.nr && dv < D) ? wvh[(int64_t)(p.r_lo + idx) * p.wv_sr + dv]
                                                 : 0.f;
          oacc[mb] = mfma(a, bw, oacc[mb]);
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
            __bf16 o4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[mb][4 * g + e] * inv_l);
            *reinterpret_cast<uint2*>(orow + dv0) = *reinterpret_cast<const uint2*>(o4);
          } else {
            float4 o4;
            o4.x = oacc[mb][4 * g + 0] * inv_l;
            o4.y = oacc[mb][4 * g + 1] * inv_l;
            o4.z = oacc[mb][4 * g + 2] * inv_l;
            o4.w = oacc[mb][4 * g + 3] * inv_l;
            *reinterpret_cast<float4*>(orow + dv0) = o4;
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
static size_t lds_bytes_t(RelMode mode, int nr, int t5_dist) {
  using G = Geo<BF16, D, NW, BC>;
  size_t extra = 0;
  if (mode == kRelShaw) extra = (size_t)G::BR * label_row_stride_impl(nr) * sizeof(float);
  if (mode == kRelT5) extra = (size_t)(2 * t5_dist + 1) * sizeof(float);
  return G::TILE_BYTES + extra;
}

constexpr int kBlockKeys = 64;  // BC for bf16
constexpr int kBlockKeysF32 = 32;

size_t lds_bytes(bool bf16, int d, const LaunchCfg& cfg, RelMode mode, bool has_wv,
                 int nr, int t5_dist) {
  (void)has_wv;
#define RELATTN_LDS(BF, DD, NWW, BCC) \
  if (bf16 == BF && d == DD && cfg.waves == NWW && cfg.kblock == BCC) \
    return lds_bytes_t<BF, DD, NWW, BCC>(mode, nr, t5_dist);
#define RELATTN_LDS_D(BF, NWW, BCC) \
  RELATTN_LDS(BF, 16, NWW, BCC) RELATTN_LDS(BF, 32, NWW, BCC) \
  RELATTN_LDS(BF, 64, NWW, BCC) RELATTN_LDS(BF, 128, NWW, BCC)
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
  const size_t lds = lds_bytes_t<BF16, D, NW, BC>((RelMode)MODE, p.nr, p.t5_dist);
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
