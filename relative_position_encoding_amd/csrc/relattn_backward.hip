// Backward of relation-aware self-attention (and of the scalar-bias arm) for
// gfx950 (CDNA4).
//
// Method: the gradients of a loss L through the forward of "Self-Attention
// with Relative Position Representations" (section 3.4, Eq. 3 and Eq. 4, with
// the split of Eq. 5) and of the T5 bias ("Relative position embeddings",
// section "T5").  With P the attention weights, dz = dL/dz and the logit
// e_ij = s q_i.(k_j + w^K_r) + b_ij (r = clip(j - i, c) + c):
//   dP_ij = dz_i.(v_j + w^V_r)        D_i = dz_i.z_i = sum_j P_ij dP_ij
//   dS_ij = P_ij (dP_ij - D_i)        (the softmax Jacobian)
//   dq_i  = s (sum_j dS_ij k_j + sum_r G[i, r] w^K_r)
//   dk_j  = s sum_i dS_ij q_i         dv_j = sum_i P_ij dz_i
//   dw^K_r = s sum_i G[i, r] q_i      dw^V_r = sum_i W[i, r] dz_i
// where G[i, r] and W[i, r] sum dS_ij and P_ij over the keys of label r; the
// bias gradient sums dS_ij over the pairs of each bucket.
//
// Three launches, no atomics (results are bitwise reproducible):
//  * bwd_q_kernel (one workgroup per 32*NW query rows, like the forward):
//    recomputes P from the forward's log-sum-exp, forms dS and accumulates dQ
//    on MFMA (dQ^T += K^T dS^T, K^T by LDS transpose reads).  Each query's
//    relative-logit row in LDS is overwritten in place by G (and W) as the
//    keys go by: inside the band every label holds exactly one key, the two
//    end labels are per-lane register sums.  The epilogue adds G W^K to dQ
//    and writes the tile's partial table gradients Q^T G and dZ^T W.  It also
//    leaves, per query, lse (log2 units), D and the relative rows for:
//  * bwd_kv_kernel (one workgroup per 32*NW key rows): a lane owns one key;
//    recomputes S = Q K^T and dP = dZ V^T per query block, and accumulates
//    dV^T += dZ^T P and dK^T += Q^T dS with MFMA.
//  * bwd_reduce_kernel: sums the partial table and bias gradients over
//    batches (and heads, for shared tables) in a fixed order.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "relattn_device.h"
#include "relattn_internal.h"
#include "relattn_tiles.h"

namespace relattn {

namespace {

constexpr float kPosInf = __builtin_inff();

template <bool BF16, int D, int NW, int BC>
struct BGeo {
  using T = std::conditional_t<BF16, __bf16, float>;
  static constexpr int ESZ = sizeof(T);
  static constexpr int BR = 32 * NW;         // rows a workgroup owns
  static constexpr int NT = 64 * NW;
  static constexpr int NKB = BC / 32;        // 32-row blocks per streamed tile
  static constexpr int DVB = (D + 31) / 32;  // 32-wide d blocks
  static constexpr int KSTEP = BF16 ? 16 : 2;
  static constexpr int NKS = D / KSTEP;
  static constexpr int ROWB = D * ESZ;
  static constexpr int TILEB = BC * ROWB;
  static constexpr int KSTR = BF16 ? 1 : 2;
};

// Waves per SIMD the register budget is sized for.
template <int D>
__host__ __device__ constexpr int bwd_waves_per_simd() {
  return D > 64 ? 1 : 2;
}

// ---- dq kernel geometry ------------------------------------------------------
// LDS: a ring of two K/V stages, then the per-query rows.  The ring also
// stages, outside the key loop, the Q and dZ tiles and the table rows.
struct LayQ {
  int ring, rg, rv, tb, tbi, gb, total;
  int lrs;       // relative row stride (floats)
  int gbs;       // bucket row stride (floats)
  int kv_chunk;  // table rows per prologue chunk (w^K and w^V side by side)
  int wk_chunk;  // w^K rows per epilogue chunk
};

template <bool BF16, int D, int NW, int BC>
__host__ __device__ inline LayQ make_lay_q(int mode, bool has_wk, bool has_wv, int nr,
                                           int t5_dist, int nb, bool want_db) {
  using G = BGeo<BF16, D, NW, BC>;
  LayQ L{};
  L.ring = 2 * 2 * G::TILEB;
  int off = L.ring;
  auto take = [&](int bytes) {
    const int at = off;
    off += (bytes + 15) & ~15;
    return at;
  };
  // a lane's reads walk a diagonal of the rows (stride lrs - 1 across lanes),
  // the epilogue reads columns (stride lrs): 2 mod 4 keeps both cheap
  L.lrs = nr + ((2 - nr) & 3);
  L.rg = L.rv = L.tb = L.tbi = L.gb = off;
  L.gbs = nb | 1;
  if (mode == kRelShaw) {
    if (has_wk) L.rg = take(G::BR * L.lrs * 4);
    if (has_wv) L.rv = take(G::BR * L.lrs * 4);
  } else if (mode == kRelT5) {
    L.tb = take((2 * t5_dist + 1) * 4);
    L.tbi = take((2 * t5_dist + 1) * 4);
    if (want_db) L.gb = take(2 * G::BR * L.gbs * 4);
  }
  L.total = off;
  L.kv_chunk = (L.ring / (2 * G::ROWB)) / 32 * 32;
  L.wk_chunk = (L.ring / G::ROWB) / 32 * 32;
  return L;
}

// ---- dk/dv kernel geometry -------------------------------------------------
// One stage: Q tile, dZ tile (BQ rows each), lse and D of the BQ queries, and
// their relative rows (nrp floats each; w^K logits, then dz.w^V).
struct LayKV {
  int q, z, lse, dd, rl, rv, stage, tb, total;
};

template <bool BF16, int D, int NW, int BQ>
__host__ __device__ inline LayKV make_lay_kv(int mode, bool has_wk, bool has_wv, int nrp,
                                             int t5_dist) {
  using G = BGeo<BF16, D, NW, BQ>;
  LayKV L{};
  int off = 0;
  auto take = [&](int bytes) {
    const int at = off;
    off += (bytes + 15) & ~15;
    return at;
  };
  L.q = take(G::TILEB);
  L.z = take(G::TILEB);
  L.lse = take(256);  // one 4-byte DMA instruction (64 lanes) each
  L.dd = take(256);
  L.rl = L.rv = off;
  if (mode == kRelShaw && has_wk) L.rl = take(BQ * nrp * 4);
  if (mode == kRelShaw && has_wv) L.rv = take(BQ * nrp * 4);
  L.stage = off;
  off = 2 * L.stage;
  // the prologue stages this workgroup's K and V rows in the ring
  off = max(off, 2 * G::BR * G::ROWB);
  L.tb = off;
  if (mode == kRelT5) take((2 * t5_dist + 1) * 4);
  L.total = off;
  return L;
}

// Workgroup id -> (b*H + h, tile).  Causal query tiles: the same dealing as
// the forward (heaviest tiles first, whole heads per XCD when they divide).
__device__ __forceinline__ void q_tile_of(int causal, int n_qtiles, int& bh, int& qt) {
  if (causal && (gridDim.x & 7) == 0 && (gridDim.x >> 3) % n_qtiles == 0) {
    const int x = blockIdx.x & 7, loc = blockIdx.x >> 3;
    const int hpx = (gridDim.x >> 3) / n_qtiles;
    const int rank = loc / hpx;
    bh = x * hpx + (loc - rank * hpx);
    qt = n_qtiles - 1 - rank;
  } else {
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    bh = lid / n_qtiles;
    qt = lid - bh * n_qtiles;
    if (causal) qt = n_qtiles - 1 - qt;
  }
}

// Flat copy of `bytes` (a multiple of 64 * size) from global to LDS with
// `size`-byte LDS-DMA requests (4 or 16), dealt to the waves.
template <int NW, int SIZE>
__device__ __forceinline__ void dma_flat(unsigned char RELATTN_LDS* lds, const void* g, int bytes,
                                         int wave, int lane) {
  constexpr int PER = 64 * SIZE;
  const int ninstr = bytes / PER;
  for (int I = wave; I < ninstr; I += NW) {
    const unsigned char* src = reinterpret_cast<const unsigned char*>(g) + I * PER + lane * SIZE;
    if constexpr (SIZE == 4) {
      __builtin_amdgcn_global_load_lds((const RELATTN_GLOBAL void*)src,
                                       (RELATTN_LDS void*)(lds + I * PER), 4, 0, 0);
    } else {
      static_assert(SIZE == 16, "4- or 16-byte requests");
      __builtin_amdgcn_global_load_lds((const RELATTN_GLOBAL void*)src,
                                       (RELATTN_LDS void*)(lds + I * PER), 16, 0, 0);
    }
  }
}

// One K/V (or Q/dZ) stage of BC rows each, row index clamped to row_max.
template <int ROWB, int NW, int BC, typename T>
__device__ __forceinline__ void stage_pair(unsigned char RELATTN_LDS* st, const T* a,
                                           int64_t a_stride, const T* b, int64_t b_stride,
                                           int row0, int row_max, int wave, int lane) {
  dma_tile<ROWB, NW>(st, a, a_stride, row0, row_max, BC, wave, lane);
  dma_tile<ROWB, NW>(st + BC * ROWB, b, b_stride, row0, row_max, BC, wave, lane);
}

template <typename T, int D>
__device__ __forceinline__ void store_row_block(T* row, const f32x16 (&acc)[(D + 31) / 32],
                                                float mul, int hh) {
#pragma unroll
  for (int mb = 0; mb < (D + 31) / 32; ++mb) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * mb + 8 * g + 4 * hh;
      if (d0 < D) {
        if constexpr (std::is_same_v<T, __bf16>) {
          bf16x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc[mb][4 * g + e] * mul);
          *reinterpret_cast<bf16x4*>(row + d0) = o4;
        } else {
          f32x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = acc[mb][4 * g + e] * mul;
          *reinterpret_cast<f32x4*>(row + d0) = o4;
        }
      }
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// dq kernel
// ---------------------------------------------------------------------------
template <int D, int NW, int BC, bool BF16, int MODE, bool HAS_WK, bool HAS_WV>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(bwd_waves_per_simd<D>()))) void bwd_q_kernel(
    const BwdParams p) {
  using G = BGeo<BF16, D, NW, BC>;
  using T = typename G::T;
  using Op = std::conditional_t<BF16, bf16x8, float>;
  constexpr int NT = G::NT, NKB = G::NKB, DVB = G::DVB, NKS = G::NKS, ROWB = G::ROWB;
  constexpr int KSTR = G::KSTR, BR = G::BR;
  constexpr bool SHAW = MODE == kRelShaw, T5 = MODE == kRelT5;
  constexpr bool ROWS = SHAW && (HAS_WK || HAS_WV);
  static_assert(2 * BR * ROWB <= 4 * G::TILEB, "Q and dZ tiles must fit the ring");

  int bh, qt;
  q_tile_of(p.causal, p.n_qtiles, bh, qt);
  const int b = bh / p.H, h = bh - b * p.H;
  const int i0 = qt * BR;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const int qrow = wave * 32 + ql;
  const int qi = i0 + qrow;
  const bool q_ok = qi < p.n;
  const int wq0 = i0 + wave * 32;
  const int c = p.clip;
  const int r_hi = p.r_lo + p.nr - 1;
  const bool want_db = T5 && p.ws_pb != nullptr;
  const int dist = p.t5_dist;

  const LayQ lay = make_lay_q<BF16, D, NW, BC>(MODE, HAS_WK, HAS_WV, p.nr, dist, p.t5.nb, want_db);
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char RELATTN_LDS* smem_lds = (unsigned char RELATTN_LDS*)smem;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem_lds;
  float* RG = reinterpret_cast<float*>(smem + lay.rg) + qrow * lay.lrs;
  float* RV = reinterpret_cast<float*>(smem + lay.rv) + qrow * lay.lrs;
  float* TB = reinterpret_cast<float*>(smem + lay.tb);
  int* TBI = reinterpret_cast<int*>(smem + lay.tbi);
  float* GB = reinterpret_cast<float*>(smem + lay.gb) + (2 * qrow + hh) * lay.gbs;

  const T* qg = reinterpret_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const T* kg = reinterpret_cast<const T*>(p.k) + b * p.k_sb + h * p.k_sh;
  const T* vg = reinterpret_cast<const T*>(p.v) + b * p.v_sb + h * p.v_sh;
  const T* og = reinterpret_cast<const T*>(p.o) + b * p.o_sb + h * p.o_sh;
  const T* zg = reinterpret_cast<const T*>(p.dout) + b * p.do_sb + h * p.do_sh;
  T* dqg = reinterpret_cast<T*>(p.dq) + b * p.dq_sb + h * p.dq_sh;
  const T* wkh = reinterpret_cast<const T*>(p.wk) + h * p.wk_sh;
  const T* wvh = reinterpret_cast<const T*>(p.wv) + h * p.wv_sh;

  // ---- Q and dZ tiles through the ring into registers (B operands)
  dma_tile<ROWB, NW>(smem_lds, qg, p.q_sn, i0, p.n - 1, BR, wave, lane);
  dma_tile<ROWB, NW>(smem_lds + BR * ROWB, zg, p.do_sn, i0, p.n - 1, BR, wave, lane);
  if constexpr (T5) {
    // log2(e) * bias and the bias entry of every offset in [-dist, dist]
    for (int x = tid; x <= 2 * dist; x += NT) {
      const int entry = p.ob ? x : t5_bucket(x - dist, p.t5);
      TB[x] = kLog2e * p.t5_bias[(entry + p.ob_lo) * p.tb_sb + h * p.tb_sh];
      TBI[x] = entry;
    }
    if (want_db) {
      float* gb0 = reinterpret_cast<float*>(smem + lay.gb);
      for (int x = tid; x < 2 * BR * lay.gbs; x += NT) gb0[x] = 0.f;
    }
  }
  float lse2 = kPosInf;  // rows past n: every weight comes out 0
  if (q_ok) lse2 = p.lse[b * p.lse_sb + h * p.lse_sh + qi] * kLog2e;
  wait_vm<0>();
  block_sync();
  Op qop[NKS], zop[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if constexpr (BF16) {
      qop[ks] = frag_row<ROWB>(smem, qrow, 2 * ks + hh);
      zop[ks] = frag_row<ROWB>(smem + BR * ROWB, qrow, 2 * ks + hh);
    } else {
      qop[ks] = elem_f32<ROWB>(smem, qrow, 2 * ks + hh);
      zop[ks] = elem_f32<ROWB>(smem + BR * ROWB, qrow, 2 * ks + hh);
    }
  }
  // D_i = dz_i . z_i (each lane half holds half of the row)
  float dd = 0.f;
  if (q_ok) {
    const T* zr = og + (int64_t)qi * p.o_sn;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (BF16) {
        const bf16x8 z8 = *reinterpret_cast<const bf16x8*>(zr + 16 * ks + 8 * hh);
#pragma unroll
        for (int e = 0; e < 8; ++e) dd = fmaf((float)z8[e], (float)zop[ks][e], dd);
      } else {
        dd = fmaf(zr[2 * ks + hh], zop[ks], dd);
      }
    }
  }
  dd = halves_sum(dd);
  if (hh == 0 && qi < p.n_pad) {
    float* st = p.ws_stat + (int64_t)bh * 2 * p.n_pad;
    st[qi] = lse2;
    st[p.n_pad + qi] = dd;
  }
  block_sync();  // the ring is free

  // ---- relative rows: Shaw row qrow holds s*log2(e)*q.w^K_r (then dS sums)
  // and dz.w^V_r (then weight sums) for labels r_lo + x, x < nr; both go to
  // the workspace for the key-side kernel
  if constexpr (ROWS) {
    const int nlb = (p.nr + 31) / 32;
    const int cb = lay.kv_chunk / 32;
    for (int lb0 = 0; lb0 < nlb; lb0 += cb) {
      const int rows = min(cb, nlb - lb0) * 32;
      if constexpr (HAS_WK)
        dma_tile<ROWB, NW>(smem_lds, wkh, p.wk_sr, p.r_lo + lb0 * 32, r_hi, rows, wave, lane);
      if constexpr (HAS_WV)
        dma_tile<ROWB, NW>(smem_lds + lay.kv_chunk * ROWB, wvh, p.wv_sr, p.r_lo + lb0 * 32, r_hi,
                           rows, wave, lane);
      wait_vm<0>();
      block_sync();
      for (int lb = lb0; lb < lb0 + rows / 32; ++lb) {
        const int row = (lb - lb0) * 32 + ql;
#pragma unroll
        for (int which = 0; which < 2; ++which) {
          if (which == 0 && !HAS_WK) continue;
          if (which == 1 && !HAS_WV) continue;
          const unsigned char* tile = smem + (which ? lay.kv_chunk * ROWB : 0);
          f32x16 acc = {};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            if constexpr (BF16) {
              acc = mfma(frag_row<ROWB>(tile, row, 2 * ks + hh), which ? zop[ks] : qop[ks], acc);
            } else {
              acc = mfma(elem_f32<ROWB>(tile, row, 2 * ks + hh), which ? zop[ks] : qop[ks], acc);
            }
          }
          const float mul = which ? 1.f : p.scale_log2;
          float* lrow = which ? RV : RG;
          float* wrow = (which ? p.ws_rv : p.ws_rl) + ((int64_t)bh * p.n_pad + qi) * p.nrp;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int x0 = lb * 32 + 8 * g + 4 * hh;  // acc[4g + e]: label x0 + e
            f32x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v4[e] = acc[4 * g + e] * mul;
              if (x0 + e < p.nr) lrow[x0 + e] = v4[e];
            }
            if (q_ok && x0 < p.nrp) *reinterpret_cast<f32x4*>(wrow + x0) = v4;
          }
        }
      }
      block_sync();  // before the next chunk or the first K/V stage
    }
  }

  // ---- key loop
  int kv_len = p.n;
  if (p.key_lens) kv_len = min(max(p.key_lens[b], 0), p.n);
  const int kv_end = p.causal ? min(kv_len, i0 + BR) : kv_len;
  const int kv_last = max(kv_len - 1, 0);
  const int ntiles = (kv_end + BC - 1) / BC;
  if (ntiles > 0)
    stage_pair<ROWB, NW, BC>(smem_lds, kg, p.k_sn, vg, p.v_sn, 0, kv_last, wave, lane);

  const int band = T5 ? dist : c;          // |delta| >= band: an end label
  const int hi_from = max(band, 1 - band);  // delta >= hi_from: the upper end
  const float rl_lo = (SHAW && HAS_WK) ? RG[0] : (T5 ? TB[0] : 0.f);
  const float rl_hi = (SHAW && HAS_WK) ? RG[p.nr - 1] : (T5 ? TB[2 * dist] : 0.f);
  const float rv_lo = (SHAW && HAS_WV) ? RV[0] : 0.f;
  const float rv_hi = (SHAW && HAS_WV) ? RV[p.nr - 1] : 0.f;
  float g_lo = 0.f, g_hi = 0.f, w_lo = 0.f, w_hi = 0.f;  // end-label sums of dS and P
  f32x16 dq[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) dq[mb] = f32x16{};
  uint32_t trb_lo[DVB], trb_hi[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) frag_col_base<ROWB, D>(32 * mb, lane, trb_lo[mb], trb_hi[mb]);
  const int hoff = BF16 ? 8 * hh : hh;

  for (int t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    wait_vm<0>();
    block_sync();  // tile t landed everywhere; stage st ^ 1 is free
    if (t + 1 < ntiles)
      stage_pair<ROWB, NW, BC>(smem_lds + (st ^ 1) * 2 * G::TILEB, kg, p.k_sn, vg, p.v_sn,
                               (t + 1) * BC, kv_last, wave, lane);
    compiler_fence();
    const int j0 = t * BC;
    if (wq0 >= p.n) continue;
    if (p.causal && j0 > wq0 + 31) continue;
    const unsigned char* Kt = smem + st * 2 * G::TILEB;
    const unsigned char* Vt = Kt + G::TILEB;

#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int jb = j0 + 32 * kb;
      if (p.causal && jb > wq0 + 31) continue;  // wave-uniform
      // S^T = K Q^T and dP^T = V dZ^T for 32 keys x this wave's 32 queries
      f32x16 s = {}, dp = {};
      const int krow = 32 * kb + k_row_of_mfma_row<BF16>(ql);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if constexpr (BF16) {
          s = mfma(frag_row<ROWB>(Kt, krow, 2 * ks + hh), qop[ks], s);
          dp = mfma(frag_row<ROWB>(Vt, krow, 2 * ks + hh), zop[ks], dp);
        } else {
          s = mfma(elem_f32<ROWB>(Kt, krow, 2 * ks + hh), qop[ks], s);
          dp = mfma(elem_f32<ROWB>(Vt, krow, 2 * ks + hh), zop[ks], dp);
        }
      }
      // register i holds key jb + hoff + ko(i), offset delta = kofs + ko(i)
      const int kofs = jb + hoff - qi;
      const int lim = min(kv_len - 1 - jb - hoff, p.causal ? -kofs : 0x3fffffff);
      const int dmin = jb - (wq0 + 31), dmax = jb + 31 - wq0;
      const bool all_lo = dmax <= -band, all_hi = dmin >= hi_from;  // wave-uniform
      float pw[16], ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ko = 16 * (i >> 3) + KSTR * (i & 7);
        const int delta = kofs + ko;
        float rl = 0.f, rv = 0.f;
        if constexpr (SHAW) {
          const int x = min(max(delta + c - p.r_lo, 0), p.nr - 1);
          if constexpr (HAS_WK) rl = all_lo ? rl_lo : (all_hi ? rl_hi : RG[x]);
          if constexpr (HAS_WV) rv = all_lo ? rv_lo : (all_hi ? rv_hi : RV[x]);
        } else if constexpr (T5) {
          rl = all_lo ? rl_lo : (all_hi ? rl_hi : TB[min(max(delta, -dist), dist) + dist]);
        }
        const bool vis = ko <= lim;
        const float pv = vis ? fast_exp2(fmaf(s[i], p.scale_log2, rl) - lse2) : 0.f;
        pw[i] = pv;
        ds[i] = vis ? pv * (dp[i] + rv - dd) : 0.f;
      }
      // per-label sums
      if constexpr (SHAW || T5) {
        if (all_lo || all_hi) {
          float gs = 0.f, ws = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            gs += ds[i];
            ws += pw[i];
          }
          if (all_lo) {
            g_lo += gs;
            w_lo += ws;
          } else {
            g_hi += gs;
            w_hi += ws;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ko = 16 * (i >> 3) + KSTR * (i & 7);
            const int delta = kofs + ko;
            if (delta <= -band) {
              g_lo += ds[i];
              w_lo += pw[i];
            } else if (delta >= hi_from) {
              g_hi += ds[i];
              w_hi += pw[i];
            } else if (q_ok && qi + delta < p.n) {
              // the only key of its label in this row (labels past the
              // reachable ones belong to masked future keys)
              if constexpr (SHAW) {
                const int x = delta + c - p.r_lo;
                if ((unsigned)x < (unsigned)p.nr) {
                  if constexpr (HAS_WK) RG[x] = ds[i];
                  if constexpr (HAS_WV) RV[x] = pw[i];
                }
              } else {
                if (want_db) GB[TBI[delta + dist]] += ds[i];
              }
            }
          }
        }
      }
      // dQ^T += K^T dS^T
      if constexpr (BF16) {
        bf16x4 klo[2 * DVB], khi[2 * DVB];
        const uint32_t kt_lds = smem_addr + (uint32_t)(Kt - smem);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb)
            frag_col_issue_blk<ROWB>(2 * kb + t2, kt_lds + trb_lo[mb], kt_lds + trb_hi[mb],
                                     klo[t2 * DVB + mb], khi[t2 * DVB + mb]);
        bf16x8 db[2];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int e = 0; e < 8; ++e) db[t2][e] = (__bf16)ds[8 * t2 + e];
        frag_col_wait(klo, khi);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb)
            dq[mb] = mfma(frag_join(klo[t2 * DVB + mb], khi[t2 * DVB + mb]), db[t2], dq[mb]);
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2)
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) {
            const int dcol = min(32 * mb + ql, D - 1);  // rows past D are never stored
            dq[mb] = mfma(elem_f32<ROWB>(Kt, 32 * kb + 2 * s2 + hh, dcol), ds[s2], dq[mb]);
          }
      }
    }
  }
  wait_vm<0>();
  block_sync();

  // ---- epilogue: final label sums of this row
  if constexpr (ROWS) {
    const float gl = halves_sum(g_lo), gh = halves_sum(g_hi);
    const float wl = halves_sum(w_lo), wh = halves_sum(w_hi);
    const int x_lo = -p.r_lo;         // label -c (present when r_lo == 0)
    const int x_hi = 2 * c - p.r_lo;  // label +c (present when < nr)
    for (int x = hh; x < p.nr; x += 2) {
      const int delta = x + p.r_lo - c;
      const int j = qi + delta;
      const bool vis = q_ok && j >= 0 && j < kv_len && (!p.causal || delta <= 0);
      float gv = 0.f, wv = 0.f;
      if (x == x_lo || x == x_hi) {
        gv = (x == x_lo ? gl : 0.f) + (x == x_hi ? gh : 0.f);
        wv = (x == x_lo ? wl : 0.f) + (x == x_hi ? wh : 0.f);
      } else if (vis) {
        if constexpr (HAS_WK) gv = RG[x];
        if constexpr (HAS_WV) wv = RV[x];
      }
      if (!q_ok) gv = wv = 0.f;
      if constexpr (HAS_WK) RG[x] = gv;
      if constexpr (HAS_WV) RV[x] = wv;
    }
    compiler_fence();  // the other half of this wave wrote the rest of the row
  }

  // ---- dQ^T += (w^K)^T G^T, w^K in label chunks through the ring
  if constexpr (SHAW && HAS_WK) {
    const int nls = (p.nr + 15) / 16;
    for (int l0 = 0; l0 < nls * 16; l0 += lay.wk_chunk) {
      const int rows = min(lay.wk_chunk, (nls * 16 - l0 + 31) / 32 * 32);
      block_sync();
      dma_tile<ROWB, NW>(smem_lds, wkh, p.wk_sr, p.r_lo + l0, r_hi, rows, wave, lane);
      wait_vm<0>();
      block_sync();
      const int ls_end = min(nls, (l0 + rows) / 16);
      for (int ls = l0 / 16; ls < ls_end; ++ls) {
        const int lsr = ls - l0 / 16;
        if constexpr (BF16) {
          bf16x8 bw;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int x = ls * 16 + 8 * hh + e;
            bw[e] = (__bf16)(x < p.nr ? RG[x] : 0.f);
          }
          bf16x4 wlo[DVB], whi[DVB];
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb)
            frag_col_issue<ROWB, D>(smem_addr, lsr * 16, 32 * mb, lane, wlo[mb], whi[mb]);
          frag_col_wait(wlo, whi);
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) dq[mb] = mfma(frag_join(wlo[mb], whi[mb]), bw, dq[mb]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int x = ls * 16 + 2 * e + hh;
            const float w = x < p.nr ? RG[x] : 0.f;
#pragma unroll
            for (int mb = 0; mb < DVB; ++mb) {
              const int dcol = min(32 * mb + ql, D - 1);
              dq[mb] = mfma(elem_f32<ROWB>(smem, lsr * 16 + 2 * e + hh, dcol), w, dq[mb]);
            }
          }
        }
      }
    }
  }
  if (q_ok) store_row_block<T, D>(dqg + (int64_t)qi * p.dq_sn, dq, p.scale, hh);

  // ---- partial table gradients of this tile: (w^K)' = s Q^T G, (w^V)' = dZ^T W
  if constexpr (ROWS) {
    block_sync();
    if constexpr (HAS_WK) dma_tile<ROWB, NW>(smem_lds, qg, p.q_sn, i0, p.n - 1, BR, wave, lane);
    if constexpr (HAS_WV)
      dma_tile<ROWB, NW>(smem_lds + BR * ROWB, zg, p.do_sn, i0, p.n - 1, BR, wave, lane);
    wait_vm<0>();
    block_sync();
    const int nlb = (p.nr + 31) / 32;
    const int per = nlb * DVB;
    constexpr int NWHICH = (HAS_WK ? 1 : 0) + (HAS_WV ? 1 : 0);
    const int64_t tile_id = (int64_t)bh * p.n_qtiles + qt;
    for (int tt = wave; tt < per * NWHICH; tt += NW) {
      const bool isv = HAS_WK ? tt >= per : true;
      const int r = (HAS_WK && isv) ? tt - per : tt;
      const int lb = r / DVB, mb = r - lb * DVB;
      const float* Gr = reinterpret_cast<const float*>(smem + (isv ? lay.rv : lay.rg));
      const unsigned char* X = smem + (isv ? BR * ROWB : 0);
      const int x = min(lb * 32 + ql, p.nr - 1);
      f32x16 acc = {};
      if constexpr (BF16) {
        const uint32_t x_lds = smem_addr + (uint32_t)(X - smem);
#pragma unroll 4
        for (int qs = 0; qs < BR / 16; ++qs) {
          bf16x4 lo[1], hi[1];
          frag_col_issue<ROWB, D>(x_lds, qs * 16, 32 * mb, lane, lo[0], hi[0]);
          bf16x8 bq;
#pragma unroll
          for (int e = 0; e < 8; ++e) bq[e] = (__bf16)Gr[(qs * 16 + 8 * hh + e) * lay.lrs + x];
          frag_col_wait(lo, hi);
          acc = mfma(frag_join(lo[0], hi[0]), bq, acc);
        }
      } else {
        const int dcol = min(32 * mb + ql, D - 1);
#pragma unroll 4
        for (int qs = 0; qs < BR / 2; ++qs)
          acc = mfma(elem_f32<ROWB>(X, 2 * qs + hh, dcol), Gr[(2 * qs + hh) * lay.lrs + x], acc);
      }
      const int lab = lb * 32 + ql;
      if (lab < p.nr) {
        float* dst = (isv ? p.ws_pv : p.ws_pk) + (tile_id * p.nr + lab) * D;
        const float mul = isv ? 1.f : p.scale;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * mb + 8 * g + 4 * hh;
          if (d0 < D) {
            f32x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = acc[4 * g + e] * mul;
            *reinterpret_cast<f32x4*>(dst + d0) = v4;
          }
        }
      }
    }
  }

  // ---- partial bias gradient of this tile (sum over its rows, fixed order)
  if constexpr (T5) {
    if (want_db) {
      GB[TBI[0]] += g_lo;
      GB[TBI[2 * dist]] += g_hi;
      block_sync();
      const float* gb0 = reinterpret_cast<const float*>(smem + lay.gb);
      const int64_t tile_id = (int64_t)bh * p.n_qtiles + qt;
      for (int e = tid; e < p.t5.nb; e += NT) {
        float acc = 0.f;
        for (int slot = 0; slot < 2 * BR; ++slot) acc += gb0[slot * lay.gbs + e];
        p.ws_pb[tile_id * p.t5.nb + e] = acc;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dk/dv kernel
// ---------------------------------------------------------------------------
template <int D, int NW, int BQ, bool BF16, int MODE, bool HAS_WK, bool HAS_WV>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(bwd_waves_per_simd<D>()))) void bwd_kv_kernel(
    const BwdParams p) {
  using G = BGeo<BF16, D, NW, BQ>;
  using T = typename G::T;
  using Op = std::conditional_t<BF16, bf16x8, float>;
  constexpr int NT = G::NT, NQB = G::NKB, DVB = G::DVB, NKS = G::NKS, ROWB = G::ROWB;
  constexpr int KSTR = G::KSTR, BR = G::BR;
  constexpr bool SHAW = MODE == kRelShaw, T5 = MODE == kRelT5;

  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / p.n_ktiles, kt = lid - bh * p.n_ktiles;
  const int b = bh / p.H, h = bh - b * p.H;
  const int k0 = kt * BR;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const int wk0 = k0 + wave * 32;
  const int kj = wk0 + ql;  // this lane's key
  const int c = p.clip;
  const int dist = p.t5_dist;

  const LayKV lay = make_lay_kv<BF16, D, NW, BQ>(MODE, HAS_WK, HAS_WV, p.nrp, dist);
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char RELATTN_LDS* smem_lds = (unsigned char RELATTN_LDS*)smem;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem_lds;
  float* TB = reinterpret_cast<float*>(smem + lay.tb);

  const T* qg = reinterpret_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const T* kg = reinterpret_cast<const T*>(p.k) + b * p.k_sb + h * p.k_sh;
  const T* vg = reinterpret_cast<const T*>(p.v) + b * p.v_sb + h * p.v_sh;
  const T* zg = reinterpret_cast<const T*>(p.dout) + b * p.do_sb + h * p.do_sh;
  T* dkg = reinterpret_cast<T*>(p.dk) + b * p.dk_sb + h * p.dk_sh;
  T* dvg = reinterpret_cast<T*>(p.dv) + b * p.dv_sb + h * p.dv_sh;
  const float* stat = p.ws_stat + (int64_t)bh * 2 * p.n_pad;
  const float* rlg = p.ws_rl + (int64_t)bh * p.n_pad * p.nrp;
  const float* rvg = p.ws_rv + (int64_t)bh * p.n_pad * p.nrp;

  // ---- this workgroup's K and V rows into registers (B operands)
  dma_tile<ROWB, NW>(smem_lds, kg, p.k_sn, k0, p.n - 1, BR, wave, lane);
  dma_tile<ROWB, NW>(smem_lds + BR * ROWB, vg, p.v_sn, k0, p.n - 1, BR, wave, lane);
  if constexpr (T5) {
    for (int x = tid; x <= 2 * dist; x += NT) {
      const int entry = p.ob ? x : t5_bucket(x - dist, p.t5);
      TB[x] = kLog2e * p.t5_bias[(entry + p.ob_lo) * p.tb_sb + h * p.tb_sh];
    }
  }
  wait_vm<0>();
  block_sync();
  Op kop[NKS], vop[NKS];
  const int krow = wave * 32 + ql;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if constexpr (BF16) {
      kop[ks] = frag_row<ROWB>(smem, krow, 2 * ks + hh);
      vop[ks] = frag_row<ROWB>(smem + BR * ROWB, krow, 2 * ks + hh);
    } else {
      kop[ks] = elem_f32<ROWB>(smem, krow, 2 * ks + hh);
      vop[ks] = elem_f32<ROWB>(smem + BR * ROWB, krow, 2 * ks + hh);
    }
  }
  block_sync();  // the ring is free

  int kv_len = p.n;
  if (p.key_lens) kv_len = min(max(p.key_lens[b], 0), p.n);
  // query tiles that can see a key of this workgroup
  const int t_lo = p.causal ? k0 / BQ : 0;
  const int t_end = (k0 < kv_len) ? (p.n + BQ - 1) / BQ : t_lo;
  auto issue = [&](int t, int stage) __attribute__((always_inline)) {
    unsigned char RELATTN_LDS* st = smem_lds + stage * lay.stage;
    const int q0 = t * BQ;
    stage_pair<ROWB, NW, BQ>(st + lay.q, qg, p.q_sn, zg, p.do_sn, q0, p.n - 1, wave, lane);
    if (wave == 0) {
      dma_flat<1, 4>(st + lay.lse, stat + q0, 256, 0, lane);
      dma_flat<1, 4>(st + lay.dd, stat + p.n_pad + q0, 256, 0, lane);
    }
    if constexpr (SHAW && HAS_WK)
      dma_flat<NW, 16>(st + lay.rl, rlg + (int64_t)q0 * p.nrp, BQ * p.nrp * 4, wave, lane);
    if constexpr (SHAW && HAS_WV)
      dma_flat<NW, 16>(st + lay.rv, rvg + (int64_t)q0 * p.nrp, BQ * p.nrp * 4, wave, lane);
    compiler_fence();
  };
  if (t_lo < t_end) issue(t_lo, 0);

  f32x16 dk[DVB], dv[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) dk[mb] = dv[mb] = f32x16{};
  uint32_t trb_lo[DVB], trb_hi[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) frag_col_base<ROWB, D>(32 * mb, lane, trb_lo[mb], trb_hi[mb]);
  const int hoff = BF16 ? 8 * hh : hh;
  const bool k_ok = kj < kv_len;

  for (int t = t_lo; t < t_end; ++t) {
    const int stg = (t - t_lo) & 1;
    wait_vm<0>();
    block_sync();
    if (t + 1 < t_end) issue(t + 1, stg ^ 1);
    const unsigned char* S0 = smem + stg * lay.stage;
    const unsigned char* Qt = S0 + lay.q;
    const unsigned char* Zt = S0 + lay.z;
    const float* LS = reinterpret_cast<const float*>(S0 + lay.lse);
    const float* DD = reinterpret_cast<const float*>(S0 + lay.dd);
    const float* RLt = reinterpret_cast<const float*>(S0 + lay.rl);
    const float* RVt = reinterpret_cast<const float*>(S0 + lay.rv);
    const int q0 = t * BQ;
    if (wk0 >= p.n || wk0 >= kv_len) continue;  // no live key in this wave

#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qb0 = q0 + 32 * qb;
      if (qb0 >= p.n) continue;
      if (p.causal && qb0 + 31 < wk0) continue;  // every query before every key
      // S = Q K^T and dP = dZ V^T: rows = queries (MFMA row order chosen so
      // that register i holds query qb0 + hoff + qo(i)), columns = keys
      f32x16 s = {}, dp = {};
      const int qrowm = 32 * qb + k_row_of_mfma_row<BF16>(ql);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if constexpr (BF16) {
          s = mfma(frag_row<ROWB>(Qt, qrowm, 2 * ks + hh), kop[ks], s);
          dp = mfma(frag_row<ROWB>(Zt, qrowm, 2 * ks + hh), vop[ks], dp);
        } else {
          s = mfma(elem_f32<ROWB>(Qt, qrowm, 2 * ks + hh), kop[ks], s);
          dp = mfma(elem_f32<ROWB>(Zt, qrowm, 2 * ks + hh), vop[ks], dp);
        }
      }
      float lsv[16], ddv[16];
      if constexpr (BF16) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int hv = 0; hv < 2; ++hv) {
            const int lq = 32 * qb + hoff + 16 * g + 4 * hv;
            const f32x4 a = *reinterpret_cast<const f32x4*>(LS + lq);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(DD + lq);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              lsv[8 * g + 4 * hv + e] = a[e];
              ddv[8 * g + 4 * hv + e] = d4[e];
            }
          }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int lq = 32 * qb + hoff + 16 * (i >> 3) + KSTR * (i & 7);
          lsv[i] = LS[lq];
          ddv[i] = DD[lq];
        }
      }
      float pw[16], ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int lq = 32 * qb + hoff + 16 * (i >> 3) + KSTR * (i & 7);
        const int qq = q0 + lq;
        const int delta = kj - qq;
        float rl = 0.f, rv = 0.f;
        if constexpr (SHAW) {
          const int x = min(max(delta + c - p.r_lo, 0), p.nr - 1);
          if constexpr (HAS_WK) rl = RLt[lq * p.nrp + x];
          if constexpr (HAS_WV) rv = RVt[lq * p.nrp + x];
        } else if constexpr (T5) {
          rl = TB[min(max(delta, -dist), dist) + dist];
        }
        const bool vis = k_ok && qq < p.n && (!p.causal || delta <= 0);
        const float pv = vis ? fast_exp2(fmaf(s[i], p.scale_log2, rl) - lsv[i]) : 0.f;
        pw[i] = pv;
        ds[i] = vis ? pv * (dp[i] + rv - ddv[i]) : 0.f;
      }
      // dV^T += dZ^T P and dK^T += Q^T dS
      if constexpr (BF16) {
        bf16x4 zlo[2 * DVB], zhi[2 * DVB], qlo[2 * DVB], qhi[2 * DVB];
        const uint32_t z_lds = smem_addr + (uint32_t)(Zt - smem);
        const uint32_t q_lds = smem_addr + (uint32_t)(Qt - smem);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) {
            frag_col_issue_blk<ROWB>(2 * qb + t2, z_lds + trb_lo[mb], z_lds + trb_hi[mb],
                                     zlo[t2 * DVB + mb], zhi[t2 * DVB + mb]);
            frag_col_issue_blk<ROWB>(2 * qb + t2, q_lds + trb_lo[mb], q_lds + trb_hi[mb],
                                     qlo[t2 * DVB + mb], qhi[t2 * DVB + mb]);
          }
        bf16x8 pb[2], db[2];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pb[t2][e] = (__bf16)pw[8 * t2 + e];
            db[t2][e] = (__bf16)ds[8 * t2 + e];
          }
        frag_col_wait(zlo, zhi);
        frag_col_wait(qlo, qhi);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) {
            dv[mb] = mfma(frag_join(zlo[t2 * DVB + mb], zhi[t2 * DVB + mb]), pb[t2], dv[mb]);
            dk[mb] = mfma(frag_join(qlo[t2 * DVB + mb], qhi[t2 * DVB + mb]), db[t2], dk[mb]);
          }
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2)
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) {
            const int dcol = min(32 * mb + ql, D - 1);
            dv[mb] = mfma(elem_f32<ROWB>(Zt, 32 * qb + 2 * s2 + hh, dcol), pw[s2], dv[mb]);
            dk[mb] = mfma(elem_f32<ROWB>(Qt, 32 * qb + 2 * s2 + hh, dcol), ds[s2], dk[mb]);
          }
      }
    }
  }
  wait_vm<0>();
  if (kj < p.n) {
    store_row_block<T, D>(dkg + (int64_t)kj * p.dk_sn, dk, p.scale, hh);
    store_row_block<T, D>(dvg + (int64_t)kj * p.dv_sn, dv, 1.f, hh);
  }
}

// ---------------------------------------------------------------------------
// Table and bias gradients: sums of the per-tile partials in a fixed order.
// blockIdx.y: 0 = d w^K, 1 = d w^V, 2 = d bias.  One thread per output.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const BwdParams p) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int which = blockIdx.y;
  const int nq = p.n_qtiles;
  if (which < 2) {
    float* out = which ? p.dwv : p.dwk;
    const float* part = which ? p.ws_pv : p.ws_pk;
    if (!out) return;
    const int ht = which ? p.htv : p.htk;
    const int nlab = 2 * p.clip + 1;
    const int64_t total = (int64_t)ht * nlab * p.d;
    if (idx >= total) return;
    const int dd = (int)(idx % p.d);
    const int r = (int)((idx / p.d) % nlab);
    const int hq = (int)(idx / ((int64_t)p.d * nlab));
    float acc = 0.f;
    const int x = r - p.r_lo;
    if (x >= 0 && x < p.nr) {
      const int h_lo = ht == 1 ? 0 : hq, h_hi = ht == 1 ? p.H : hq + 1;
      for (int b = 0; b < p.B; ++b)
        for (int hh = h_lo; hh < h_hi; ++hh) {
          const float* src = part + ((int64_t)(b * p.H + hh) * nq * p.nr + x) * p.d + dd;
          for (int t = 0; t < nq; ++t) acc += src[(int64_t)t * p.nr * p.d];
        }
    }
    const int64_t sh = which ? p.dwv_sh : p.dwk_sh, sr = which ? p.dwv_sr : p.dwk_sr;
    out[hq * sh + r * sr + dd] = acc;
  } else {
    if (!p.db) return;
    const int nbt = p.t5.nb;  // entries per head in the partials
    if (p.ob) {
      // offset-bias table [hb, 2W + 1]: entries outside the loaded window
      // (offsets no pair reaches) get zero
      const int nw = 2 * p.ob_w + 1;
      const int64_t total = (int64_t)p.hb * nw;
      if (idx >= total) return;
      const int w = (int)(idx % nw), hq = (int)(idx / nw);
      const int e = w - p.ob_lo;
      float acc = 0.f;
      if (e >= 0 && e < nbt) {
        const int h_lo = p.hb == 1 ? 0 : hq, h_hi = p.hb == 1 ? p.H : hq + 1;
        for (int b = 0; b < p.B; ++b)
          for (int hh = h_lo; hh < h_hi; ++hh) {
            const float* src = p.ws_pb + (int64_t)(b * p.H + hh) * nq * nbt + e;
            for (int t = 0; t < nq; ++t) acc += src[(int64_t)t * nbt];
          }
      }
      p.db[hq * p.db_s0 + w * p.db_s1] = acc;
    } else {
      // T5 table [nb, H]
      const int64_t total = (int64_t)nbt * p.H;
      if (idx >= total) return;
      const int hq = (int)(idx % p.H), e = (int)(idx / p.H);
      float acc = 0.f;
      for (int b = 0; b < p.B; ++b) {
        const float* src = p.ws_pb + (int64_t)(b * p.H + hq) * nq * nbt + e;
        for (int t = 0; t < nq; ++t) acc += src[(int64_t)t * nbt];
      }
      p.db[e * p.db_s0 + hq * p.db_s1] = acc;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: LDS sizes and launch dispatch.
// ---------------------------------------------------------------------------
// dq kernel: keys per tile, and waves (32 query rows each) for the wide
// shape and for the narrow one that halves the per-query LDS rows; dk/dv
// kernel: waves (32 keys each), and queries per tile, wide and narrow.
template <bool BF16, int D>
struct BwdShape {
  static constexpr bool BIG = BF16 && D <= 64;
  static constexpr int QBC = BIG ? 64 : 32;
  static constexpr int QW_WIDE = BIG ? 4 : 2;
  static constexpr int QW_NARROW = QW_WIDE / 2;
  static constexpr int KW = BF16 ? 4 : 2;
  static constexpr int KBQ_WIDE = BIG ? 64 : 32;
  static constexpr int KBQ_NARROW = 32;
};

template <bool BF16, int D>
static size_t lds_q_t(int qwaves, RelMode mode, bool has_wk, bool has_wv, int nr, int t5_dist,
                      int nb, bool want_db) {
  using S = BwdShape<BF16, D>;
  if (qwaves == S::QW_WIDE)
    return (size_t)make_lay_q<BF16, D, S::QW_WIDE, S::QBC>(mode, has_wk, has_wv, nr, t5_dist, nb,
                                                           want_db)
        .total;
  return (size_t)make_lay_q<BF16, D, S::QW_NARROW, S::QBC>(mode, has_wk, has_wv, nr, t5_dist, nb,
                                                           want_db)
      .total;
}
template <bool BF16, int D>
static size_t lds_kv_t(int kqblock, RelMode mode, bool has_wk, bool has_wv, int nrp,
                       int t5_dist) {
  using S = BwdShape<BF16, D>;
  if (kqblock == S::KBQ_WIDE)
    return (size_t)make_lay_kv<BF16, D, S::KW, S::KBQ_WIDE>(mode, has_wk, has_wv, nrp, t5_dist)
        .total;
  return (size_t)make_lay_kv<BF16, D, S::KW, S::KBQ_NARROW>(mode, has_wk, has_wv, nrp, t5_dist)
      .total;
}

template <bool BF16, int D>
static BwdCfg cfg_t(bool narrow_q, bool narrow_kv) {
  using S = BwdShape<BF16, D>;
  return BwdCfg{narrow_q ? S::QW_NARROW : S::QW_WIDE, S::QBC, S::KW,
                narrow_kv ? S::KBQ_NARROW : S::KBQ_WIDE};
}

BwdCfg bwd_cfg(bool bf16, int d, bool narrow_q, bool narrow_kv) {
  if (bf16) {
    if (d > 64) return cfg_t<true, 128>(narrow_q, narrow_kv);
    return cfg_t<true, 64>(narrow_q, narrow_kv);
  }
  return cfg_t<false, 64>(narrow_q, narrow_kv);
}

template <bool BF16>
static size_t lds_q_d(int d, int qw, RelMode mode, bool wk, bool wv, int nr, int dist, int nb,
                      bool db) {
  switch (d) {
    case 16: return lds_q_t<BF16, 16>(qw, mode, wk, wv, nr, dist, nb, db);
    case 32: return lds_q_t<BF16, 32>(qw, mode, wk, wv, nr, dist, nb, db);
    case 64: return lds_q_t<BF16, 64>(qw, mode, wk, wv, nr, dist, nb, db);
    default: return lds_q_t<BF16, 128>(qw, mode, wk, wv, nr, dist, nb, db);
  }
}
template <bool BF16>
static size_t lds_kv_d(int d, int bq, RelMode mode, bool wk, bool wv, int nrp, int dist) {
  switch (d) {
    case 16: return lds_kv_t<BF16, 16>(bq, mode, wk, wv, nrp, dist);
    case 32: return lds_kv_t<BF16, 32>(bq, mode, wk, wv, nrp, dist);
    case 64: return lds_kv_t<BF16, 64>(bq, mode, wk, wv, nrp, dist);
    default: return lds_kv_t<BF16, 128>(bq, mode, wk, wv, nrp, dist);
  }
}

size_t bwd_lds_q(bool bf16, int d, const BwdCfg& cfg, RelMode mode, bool has_wk, bool has_wv,
                 int nr, int t5_dist, int nb, bool want_db) {
  return bf16 ? lds_q_d<true>(d, cfg.qwaves, mode, has_wk, has_wv, nr, t5_dist, nb, want_db)
              : lds_q_d<false>(d, cfg.qwaves, mode, has_wk, has_wv, nr, t5_dist, nb, want_db);
}
size_t bwd_lds_kv(bool bf16, int d, const BwdCfg& cfg, RelMode mode, bool has_wk, bool has_wv,
                  int nrp, int t5_dist) {
  return bf16 ? lds_kv_d<true>(d, cfg.kqblock, mode, has_wk, has_wv, nrp, t5_dist)
              : lds_kv_d<false>(d, cfg.kqblock, mode, has_wk, has_wv, nrp, t5_dist);
}

template <int D, int NW, int BC, bool BF16, int MODE, bool WK, bool WV>
static int launch_q(const BwdParams& p, hipStream_t s) {
  const bool want_db = MODE == kRelT5 && p.ws_pb != nullptr;
  const LayQ lay = make_lay_q<BF16, D, NW, BC>(MODE, WK, WV, p.nr, p.t5_dist, p.t5.nb, want_db);
  auto kern = bwd_q_kernel<D, NW, BC, BF16, MODE, WK, WV>;
  if (lay.total > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             lay.total);
    if (e != hipSuccess) return (int)e;
  }
  const dim3 grid((unsigned)((int64_t)p.B * p.H * p.n_qtiles));
  hipLaunchKernelGGL(kern, grid, dim3(64 * NW), (size_t)lay.total, s, p);
  return (int)hipGetLastError();
}

template <int D, int NW, int BQ, bool BF16, int MODE, bool WK, bool WV>
static int launch_kv(const BwdParams& p, hipStream_t s) {
  const LayKV lay = make_lay_kv<BF16, D, NW, BQ>(MODE, WK, WV, p.nrp, p.t5_dist);
  auto kern = bwd_kv_kernel<D, NW, BQ, BF16, MODE, WK, WV>;
  if (lay.total > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             lay.total);
    if (e != hipSuccess) return (int)e;
  }
  const dim3 grid((unsigned)((int64_t)p.B * p.H * p.n_ktiles));
  hipLaunchKernelGGL(kern, grid, dim3(64 * NW), (size_t)lay.total, s, p);
  return (int)hipGetLastError();
}

template <bool BF16, int D, int MODE, bool WK, bool WV>
static int launch_bwd_t(const BwdCfg& cfg, const BwdParams& p, void* stream) {
  using S = BwdShape<BF16, D>;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int e = cfg.qwaves == S::QW_WIDE
              ? launch_q<D, S::QW_WIDE, S::QBC, BF16, MODE, WK, WV>(p, s)
              : launch_q<D, S::QW_NARROW, S::QBC, BF16, MODE, WK, WV>(p, s);
  if (e != (int)hipSuccess) return e;
  e = cfg.kqblock == S::KBQ_WIDE ? launch_kv<D, S::KW, S::KBQ_WIDE, BF16, MODE, WK, WV>(p, s)
                                 : launch_kv<D, S::KW, S::KBQ_NARROW, BF16, MODE, WK, WV>(p, s);
  if (e != (int)hipSuccess) return e;
  if (p.dwk || p.dwv || p.db) {
    int64_t most = 0;
    if (p.dwk) most = max(most, (int64_t)p.htk * (2 * p.clip + 1) * p.d);
    if (p.dwv) most = max(most, (int64_t)p.htv * (2 * p.clip + 1) * p.d);
    if (p.db) most = max(most, p.ob ? (int64_t)p.hb * (2 * p.ob_w + 1) : (int64_t)p.t5.nb * p.H);
    const dim3 grid((unsigned)((most + 255) / 256), 3);
    hipLaunchKernelGGL(bwd_reduce_kernel, grid, dim3(256), 0, s, p);
    e = (int)hipGetLastError();
  }
  return e;
}

template <bool BF16, int D>
static int launch_bwd_mode(const BwdCfg& c, RelMode mode, bool wk, bool wv, const BwdParams& p,
                           void* stream) {
  if (mode == kRelT5) return launch_bwd_t<BF16, D, kRelT5, false, false>(c, p, stream);
  if (mode == kRelShaw) {
    if (wk && wv) return launch_bwd_t<BF16, D, kRelShaw, true, true>(c, p, stream);
    if (wk) return launch_bwd_t<BF16, D, kRelShaw, true, false>(c, p, stream);
    return launch_bwd_t<BF16, D, kRelShaw, false, true>(c, p, stream);
  }
  return launch_bwd_t<BF16, D, kRelNone, false, false>(c, p, stream);
}

template <bool BF16>
static int launch_bwd_d(int d, const BwdCfg& c, RelMode mode, bool wk, bool wv,
                        const BwdParams& p, void* stream) {
  switch (d) {
    case 16: return launch_bwd_mode<BF16, 16>(c, mode, wk, wv, p, stream);
    case 32: return launch_bwd_mode<BF16, 32>(c, mode, wk, wv, p, stream);
    case 64: return launch_bwd_mode<BF16, 64>(c, mode, wk, wv, p, stream);
    default: return launch_bwd_mode<BF16, 128>(c, mode, wk, wv, p, stream);
  }
}

int launch_bwd(bool bf16, int d, const BwdCfg& cfg, RelMode mode, bool has_wk, bool has_wv,
               const BwdParams& p, void* stream) {
  return bf16 ? launch_bwd_d<true>(d, cfg, mode, has_wk, has_wv, p, stream)
              : launch_bwd_d<false>(d, cfg, mode, has_wk, has_wv, p, stream);
}

}  // namespace relattn
