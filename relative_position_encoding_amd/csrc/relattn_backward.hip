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
// Two launches, no atomics (results are bitwise reproducible):
//  * bwd_q_kernel (one workgroup per 32*NW query rows, like the forward):
//    recomputes P from the forward's log-sum-exp, forms dS and accumulates dQ
//    on MFMA (dQ^T += K^T dS^T, K^T by LDS transpose reads).  Each query's
//    relative-logit row in LDS is overwritten in place by G (and W) as the
//    keys go by: inside the band every label holds exactly one key, the two
//    end labels are per-lane register sums.  The epilogue adds G W^K to dQ
//    and writes the tile's partial table gradients Q^T G and dZ^T W.  It also
//    leaves, per query, lse (log2 units) and D for:
//  * bwd_kv_kernel (one workgroup per 32*NW key rows): a lane owns one key;
//    recomputes S = Q K^T and dP = dZ V^T per query block, and accumulates
//    dV^T += dZ^T P and dK^T += Q^T dS with MFMA.  The relative rows of each
//    query tile are recomputed there too (one small MFMA product against the
//    table rows held in LDS) rather than read back from memory.
//  * after their own keys, the dk/dv workgroups (under the causal mask the
//    lightest ones) sum the partial table and bias gradients over batches
//    (and heads, for shared tables) in a fixed order.
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
  // A lane's logits come in groups of 8 keys KSTR apart, spanning SPAN
  // offsets.  The dq kernel's relative rows hold the reachable labels with
  // PADL entries below and PADU above, so that a group reads and writes its 8
  // entries from one base (clamped into the row) without a per-key test.
  static constexpr int SPAN = 7 * KSTR + 1;
  static constexpr int PADL = SPAN - 1;
  static constexpr int PADU = SPAN - 1;
};

// Waves per SIMD the register budget is sized for.
template <int D>
__host__ __device__ constexpr int bwd_waves_per_simd() {
  return D > 64 ? 1 : 2;
}

// ---- dq kernel geometry ------------------------------------------------------
// LDS: a ring of two K/V stages (in the epilogue it takes the Q and dZ
// tiles), the table rows of the reachable labels (resident), then the
// per-query rows (Shaw) or the offset vector and bucket rows (T5).
struct LayQ {
  int ring, tk, tv, rg, rv, tb, tbi, gb, gw, xs, total;
  int lrs;       // relative row stride (floats)
  int gbs;       // bucket row stride (floats)
  int tab_rows;  // table rows held (labels rounded up to 32)
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
  {
    const int m = nr + G::PADL + G::PADU;
    L.lrs = m + ((2 - m) & 3);
  }
  L.tab_rows = (nr + 31) / 32 * 32;
  L.tk = L.tv = L.rg = L.rv = L.tb = L.tbi = L.gb = L.gw = L.xs = off;
  L.gbs = (mode == kRelGraph ? nr : nb) | 1;
  if (mode == kRelShaw || mode == kRelXL || mode == kRelGraph) {
    if (has_wk) {
      L.tk = take(L.tab_rows * G::ROWB);
      L.rg = take(G::BR * L.lrs * 4);
    }
    if (has_wv) {
      L.tv = take(L.tab_rows * G::ROWB);
      L.rv = take(G::BR * L.lrs * 4);
    }
    if (mode == kRelGraph) {
      // edge labels repeat along a row: per query and lane half, the sums of
      // dS (key table) and of P (value table) by label
      if (has_wk) L.gb = take(2 * G::BR * L.gbs * 4);
      if (has_wv) L.gw = take(2 * G::BR * L.gbs * 4);
    }
  } else if (mode == kRelT5) {
    L.tb = take((2 * t5_dist + 1) * 4);
    L.tbi = take((2 * t5_dist + 1) * 4);
    if (want_db) L.gb = take(2 * G::BR * L.gbs * 4);
  } else if (mode == kRelGrid) {
    // the head's table, and one bias-gradient row per wave and lane half
    L.tb = take(nb * 4);
    if (want_db) L.gb = take(2 * NW * L.gbs * 4);
  } else if (mode == kRelLabel) {
    // the head's table, and one bias-gradient row per query and lane half
    L.tb = take(nb * 4);
    if (want_db) L.gb = take(2 * G::BR * L.gbs * 4);
  }
  // Transformer-XL: per wave, its rows' sums of a dq-shaped accumulator
  if (mode == kRelXL) L.xs = take(NW * D * 4);
  L.total = off;
  return L;
}

// Row fragments of one row as the B operand of a 32x32 MFMA (lane half hh
// holds columns 16 ks + 8 hh + 0..7 for bf16, 2 ks + hh for fp32), read
// straight from memory.
template <bool BF16, int D, typename Op, typename T>
__device__ __forceinline__ void load_row_frags(const T* row, int hh, Op (&op)[BF16 ? D / 16 : D / 2]) {
#pragma unroll
  for (int ks = 0; ks < (BF16 ? D / 16 : D / 2); ++ks) {
    if constexpr (BF16) {
      op[ks] = *reinterpret_cast<const bf16x8*>(row + 16 * ks + 8 * hh);
    } else {
      op[ks] = row[2 * ks + hh];
    }
  }
}

// ---- dk/dv kernel geometry -------------------------------------------------
// A ring of two stages, each: the Q and dZ tiles (BQ rows each) and the lse
// and D of the BQ queries.  Then, for the Shaw tables: the table rows of the
// reachable labels (resident), the tile's relative rows (its queries'
// s*log2(e)*q.w^K_r and dz.w^V_r, computed per tile) and, per query, the two
// end labels' values less lse and D.
struct LayKV {
  int q, z, lse, dd, stage, rl, rv, tail, tk, tv, tb, xb, total;
  int lrs;       // relative row stride (floats)
  int tab_rows;  // table rows held (labels rounded up to 32)
};

template <bool BF16, int D, int NW, int BQ>
__host__ __device__ inline LayKV make_lay_kv(int mode, bool has_wk, bool has_wv, int nr,
                                             int t5_dist, int nb) {
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
  L.stage = off;
  off = 2 * L.stage;
  L.lrs = nr + ((2 - nr) & 3);
  L.tab_rows = (nr + 31) / 32 * 32;
  L.rl = L.rv = L.tail = L.tk = L.tv = L.tb = L.xb = off;
  if ((mode == kRelShaw || mode == kRelXL || mode == kRelGraph) && (has_wk || has_wv)) {
    if (has_wk) {
      L.tk = take(L.tab_rows * G::ROWB);
      L.rl = take(BQ * L.lrs * 4);
    }
    if (has_wv) {
      L.tv = take(L.tab_rows * G::ROWB);
      L.rv = take(BQ * L.lrs * 4);
    }
    L.tail = take(4 * BQ * 4);
  }
  if (mode == kRelT5) L.tb = take((2 * t5_dist + 1) * 4);
  if (mode == kRelGrid || mode == kRelLabel) L.tb = take(nb * 4);  // the head's table
  // Transformer-XL: v . R_r of every table row
  if (mode == kRelXL) L.xb = take(L.tab_rows * 4);
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
// Returns the number of DMA instructions this wave issued.
template <int ROWB, int NW, int BC, typename T>
__device__ __forceinline__ int stage_pair(unsigned char RELATTN_LDS* st, const T* a,
                                          int64_t a_stride, const T* b, int64_t b_stride,
                                          int row0, int row_max, int wave, int lane) {
  return dma_tile<ROWB, NW>(st, a, a_stride, row0, row_max, BC, wave, lane) +
         dma_tile<ROWB, NW>(st + BC * ROWB, b, b_stride, row0, row_max, BC, wave, lane);
}

template <typename T, int D>
__device__ __forceinline__ void store_row_block(T* row, const f32x16 (&acc)[(D + 31) / 32],
                                                float mul, int hh, bool zero = false) {
#pragma unroll
  for (int mb = 0; mb < (D + 31) / 32; ++mb) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * mb + 8 * g + 4 * hh;
      if (d0 < D) {
        if constexpr (std::is_same_v<T, __bf16>) {
          bf16x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(zero ? 0.f : acc[mb][4 * g + e] * mul);
          *reinterpret_cast<bf16x4*>(row + d0) = o4;
        } else {
          f32x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = zero ? 0.f : acc[mb][4 * g + e] * mul;
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
  // Transformer-XL runs the key-table path with R as the table; the tables
  // by edge label (GRAPH) run it with each pair's label as its table row
  constexpr bool XL = MODE == kRelXL, GRAPH = MODE == kRelGraph;
  constexpr bool SHAW = MODE == kRelShaw || XL || GRAPH, T5 = MODE == kRelT5;
  constexpr bool GRID = MODE == kRelGrid, LAB = MODE == kRelLabel;
  constexpr bool ROWS = SHAW && (HAS_WK || HAS_WV);
  static_assert(2 * BR * ROWB <= 4 * G::TILEB, "Q and dZ tiles must fit the ring");
  constexpr int SPAN = G::SPAN, PADL = G::PADL;

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
  const bool want_db = (T5 || GRID || LAB) && p.ws_pb != nullptr;
  const int dist = p.t5_dist;

  const LayQ lay = make_lay_q<BF16, D, NW, BC>(MODE, HAS_WK, HAS_WV, p.nr, dist, p.t5.nb, want_db);
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char RELATTN_LDS* smem_lds = (unsigned char RELATTN_LDS*)smem;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem_lds;
  // this query's rows; entry PADL + x holds label r_lo + x
  float* RGp = reinterpret_cast<float*>(smem + lay.rg) + qrow * lay.lrs;
  float* RVp = reinterpret_cast<float*>(smem + lay.rv) + qrow * lay.lrs;
  float* RG = RGp + PADL;
  float* RV = RVp + PADL;
  float* TB = reinterpret_cast<float*>(smem + lay.tb);
  int* TBI = reinterpret_cast<int*>(smem + lay.tbi);
  // T5: a bias-gradient row per query and lane half; 2-D window: per wave and
  // lane half (within one register, the 32 lanes of a half hold one key and 32
  // queries, whose 2-D offsets are all different, so their updates never meet)
  float* GB = reinterpret_cast<float*>(smem + lay.gb) +
              (GRID ? 2 * wave + hh : 2 * qrow + hh) * lay.gbs;

  const T* qg = reinterpret_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const T* kg = reinterpret_cast<const T*>(p.k) + b * p.k_sb + h * p.k_sh;
  const T* vg = reinterpret_cast<const T*>(p.v) + b * p.v_sb + h * p.v_sh;
  const T* og = reinterpret_cast<const T*>(p.o) + b * p.o_sb + h * p.o_sh;
  const T* zg = reinterpret_cast<const T*>(p.dout) + b * p.do_sb + h * p.do_sh;
  T* dqg = reinterpret_cast<T*>(p.dq) + b * p.dq_sb + h * p.dq_sh;
  const T* wkh = reinterpret_cast<const T*>(p.wk) + h * p.wk_sh;
  const T* wvh = reinterpret_cast<const T*>(p.wv) + h * p.wv_sh;
  [[maybe_unused]] const uint8_t* labg = (LAB || GRAPH) ? p.lab + b * p.lab_sb : nullptr;
  // edge-label tables: this lane's rows of label sums (dS, P)
  [[maybe_unused]] float* GSr = reinterpret_cast<float*>(smem + lay.gb) + (2 * qrow + hh) * lay.gbs;
  [[maybe_unused]] float* GWr = reinterpret_cast<float*>(smem + lay.gw) + (2 * qrow + hh) * lay.gbs;

  // ---- everything the loop needs, requested at once: this lane's q and dz
  // row (B operands, straight from memory), the lse, z for D, the table rows
  // (LDS, resident) or the bias window, and the first K/V tile
  int kv_len = p.n;
  if (p.key_lens) kv_len = min(max(p.key_lens[b], 0), p.n);
  const int kv_end = p.causal ? min(kv_len, i0 + BR) : kv_len;
  const int kv_last = max(kv_len - 1, 0);
  const int ntiles = (kv_end + BC - 1) / BC;
  const int qr = min(qi, p.n - 1);
  Op qop[NKS], zop[NKS];
  load_row_frags<BF16, D>(qg + (int64_t)qr * p.q_sn, hh, qop);
  load_row_frags<BF16, D>(zg + (int64_t)qr * p.do_sn, hh, zop);
  Op oop[NKS];
  load_row_frags<BF16, D>(og + (int64_t)qr * p.o_sn, hh, oop);
  // Transformer-XL: the head's global biases u (content logit) and v
  // (relative logit), in the layout of the q fragments
  [[maybe_unused]] Op xu[NKS], xv[NKS];
  if constexpr (XL) {
    load_row_frags<BF16, D>(reinterpret_cast<const T*>(p.xl_u) + h * p.xl_u_sh, hh, xu);
    load_row_frags<BF16, D>(reinterpret_cast<const T*>(p.xl_v) + h * p.xl_v_sh, hh, xv);
  }
  float lse2 = kPosInf;  // rows past n: every weight comes out 0
  if (q_ok) lse2 = p.lse[b * p.lse_sb + h * p.lse_sh + qi] * kLog2e;
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
  if constexpr (GRAPH) {
    for (int x = tid; x < 2 * BR * lay.gbs; x += NT) {
      if constexpr (HAS_WK) reinterpret_cast<float*>(smem + lay.gb)[x] = 0.f;
      if constexpr (HAS_WV) reinterpret_cast<float*>(smem + lay.gw)[x] = 0.f;
    }
  }
  if constexpr (GRID || LAB) {
    // log2(e) * the head's (2M - 1)^2 or NL entries
    for (int x = tid; x < p.t5.nb; x += NT)
      TB[x] = kLog2e * p.t5_bias[x * p.tb_sb + h * p.tb_sh];
    if (want_db) {
      float* gb0 = reinterpret_cast<float*>(smem + lay.gb);
      for (int x = tid; x < (GRID ? 2 * NW : 2 * BR) * lay.gbs; x += NT) gb0[x] = 0.f;
    }
  }
  compiler_fence();
  if constexpr (SHAW && HAS_WK)
    dma_tile<ROWB, NW>(smem_lds + lay.tk, wkh, p.wk_sr, p.r_lo, r_hi, lay.tab_rows, wave, lane);
  if constexpr (SHAW && HAS_WV)
    dma_tile<ROWB, NW>(smem_lds + lay.tv, wvh, p.wv_sr, p.r_lo, r_hi, lay.tab_rows, wave, lane);
  constexpr int STAGEB = 2 * G::TILEB;
  if (ntiles > 0)
    stage_pair<ROWB, NW, BC>(smem_lds, kg, p.k_sn, vg, p.v_sn, 0, kv_last, wave, lane);
  compiler_fence();
  // D_i = dz_i . z_i (each lane half holds half of the row)
  float dd = 0.f;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if constexpr (BF16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) dd = fmaf((float)oop[ks][e], (float)zop[ks][e], dd);
    } else {
      dd = fmaf(oop[ks], zop[ks], dd);
    }
  }
  dd = halves_sum(q_ok ? dd : 0.f);
  if (hh == 0 && qi < p.n_pad) {
    float* st = p.ws_stat + (int64_t)bh * 2 * p.n_pad;
    st[qi] = lse2;
    st[p.n_pad + qi] = dd;
  }
  wait_vm<0>();
  block_sync();  // tables, bias window and the first K/V tile landed

  // ---- relative rows: Shaw row qrow holds s*log2(e)*q.w^K_r (then dS sums)
  // and dz.w^V_r (then weight sums) for labels r_lo + x, x < nr
  if constexpr (ROWS) {
    // the key table's product takes q + v under Transformer-XL
    Op qrel[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qrel[ks] = XL ? op_add(qop[ks], xv[ks]) : qop[ks];
    const int nlb = lay.tab_rows / 32;
    for (int lb = 0; lb < nlb; ++lb) {
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        if (which == 0 && !HAS_WK) continue;
        if (which == 1 && !HAS_WV) continue;
        const unsigned char* tile = smem + (which ? lay.tv : lay.tk);
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if constexpr (BF16) {
            acc = mfma(frag_row<ROWB>(tile, lb * 32 + ql, 2 * ks + hh), which ? zop[ks] : qrel[ks],
                       acc);
          } else {
            acc = mfma(elem_f32<ROWB>(tile, lb * 32 + ql, 2 * ks + hh), which ? zop[ks] : qrel[ks],
                       acc);
          }
        }
        const float mul = which ? 1.f : p.scale_log2;
        float* lrow = which ? RV : RG;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int x = lb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);  // label of acc[i]
          if (x < p.nr) lrow[x] = acc[i] * mul;
        }
      }
    }
    compiler_fence();  // each row is read back by the lanes of its own wave only
  }
  // Transformer-XL: the content logits take q + u
  if constexpr (XL) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qop[ks] = op_add(qop[ks], xu[ks]);
  }

  // ---- key loop (tile 0 is in stage 0)
  // |delta| >= band: an end label (none in the 2-D window or by edge label:
  // every pair has its own entry)
  const int band = T5 ? dist : ((GRID || LAB || GRAPH) ? (1 << 30) : c);
  const int hi_from = max(band, 1 - band);  // delta >= hi_from: the upper end
  const float rl_lo = (SHAW && HAS_WK) ? RG[0] : (T5 ? TB[0] : 0.f);
  const float rl_hi = (SHAW && HAS_WK) ? RG[p.nr - 1] : (T5 ? TB[2 * dist] : 0.f);
  const float rv_lo = (SHAW && HAS_WV) ? RV[0] : 0.f;
  const float rv_hi = (SHAW && HAS_WV) ? RV[p.nr - 1] : 0.f;
  // running sums of dS and P over every key, and over the keys of the upper
  // end label (the lower end's sum is what the in-band and upper sums leave)
  float g_all = 0.f, g_hi = 0.f, w_all = 0.f, w_hi = 0.f;
  float g_lo = 0.f;  // T5: lower end bucket's sum of dS
  // in-band offsets whose label is reachable: their group is stored whole
  const int wb_lo = max(1, p.r_lo) - c, wb_hi = min(2 * c - 1, r_hi) - c;
  const int dlo = p.r_lo - c;  // offset of label entry 0
  f32x16 dq[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) dq[mb] = f32x16{};
  uint32_t trb_lo[DVB], trb_hi[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) frag_col_base<ROWB, D>(32 * mb, lane, trb_lo[mb], trb_hi[mb]);
  const int hoff = BF16 ? 8 * hh : hh;

  for (int t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    if (t > 0) {
      wait_vm<0>();
      block_sync();  // tile t landed everywhere; the other stage is free
    }
    if (t + 1 < ntiles)
      stage_pair<ROWB, NW, BC>(smem_lds + (st ^ 1) * STAGEB, kg, p.k_sn, vg, p.v_sn,
                               (t + 1) * BC, kv_last, wave, lane);
    compiler_fence();
    const int j0 = t * BC;
    if (wq0 >= p.n) continue;
    if (p.causal && j0 > wq0 + 31) continue;
    const unsigned char* Kt = smem + st * STAGEB;
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
      // wave-uniform: the whole block at one end label (or no relative term)
      const bool all_lo = dmax <= -band, all_hi = dmin >= hi_from;
      const bool off_band = MODE == kRelNone || all_lo || all_hi;
      // some key of the block hidden from some query of the wave
      const bool need_mask = jb + 31 >= kv_len || (p.causal && jb + 31 > wq0);
      float pw[16], ds[16];
      if (off_band) {
        // one relative logit and one value term for every key of the block:
        // P = 2^(s*log2e*S + (L_end - lse)), dS = P (dP + (V_end - D))
        const float cl = (all_hi ? rl_hi : rl_lo) - lse2;
        const float cv = (all_hi ? rv_hi : rv_lo) - dd;
        auto run = [&](auto mask_tag) __attribute__((always_inline)) {
          constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float pv = fast_exp2(fmaf(s[i], p.scale_log2, cl));
            if constexpr (MASK) pv = (16 * (i >> 3) + KSTR * (i & 7) <= lim) ? pv : 0.f;
            pw[i] = pv;
            ds[i] = pv * (dp[i] + cv);
          }
        };
        if (need_mask) {
          run(std::true_type{});
        } else {
          run(std::false_type{});
        }
        if constexpr (SHAW || T5) {
          float gs = 0.f, ws = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            gs += ds[i];
            ws += pw[i];
          }
          if constexpr (SHAW) {
            g_all += gs;
            w_all += ws;
          }
          if (all_hi) {
            g_hi += gs;
            w_hi += ws;
          } else if constexpr (T5) {
            g_lo += gs;
          }
        }
      } else if constexpr (GRAPH) {
        // tables by edge label: each key's relative logit and value term from
        // its label's entries of this query's rows; the key's dS and P go to
        // the label's sums in this lane's own rows (labels repeat along a row)
        const uint8_t* lrow = labg + (int64_t)min(qi, p.n - 1) * p.lab_sn;
        const int cmax = ((p.n + 15) & ~15) - 16;
        uint4 ch[2];
#pragma unroll
        for (int g = 0; g < 2; ++g)
          ch[g] = *reinterpret_cast<const uint4*>(lrow + min(jb + 16 * g, cmax));
        int ent[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint4 c4 = ch[i >> 3];
          const int e = i & 7;
          uint32_t lb;
          if constexpr (BF16) {
            const uint32_t w = (e >> 2) ? (hh ? c4.w : c4.y) : (hh ? c4.z : c4.x);
            lb = (w >> (8 * (e & 3))) & 0xffu;
          } else {
            const uint32_t w = (e >> 1) == 0 ? c4.x : (e >> 1) == 1 ? c4.y
                             : (e >> 1) == 2 ? c4.z : c4.w;
            lb = (w >> (8 * (2 * (e & 1) + hh))) & 0xffu;
          }
          ent[i] = min((int)lb, p.nr - 1);  // a label past the tables reads their last row
          const int ko = 16 * (i >> 3) + KSTR * (i & 7);
          const bool vis = ko <= lim;
          const float rl = HAS_WK ? RG[ent[i]] : 0.f;
          const float rv = HAS_WV ? RV[ent[i]] : 0.f;
          float ex = fast_exp2(fmaf(s[i], p.scale_log2, rl) - lse2);
          asm volatile("" : "+v"(ex));
          const float pv = vis ? ex : 0.f;
          pw[i] = pv;
          ds[i] = vis ? pv * (dp[i] + rv - dd) : 0.f;
        }
        if (q_ok) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if constexpr (HAS_WK) GSr[ent[i]] += ds[i];
            if constexpr (HAS_WV) GWr[ent[i]] += pw[i];
          }
        }
      } else if constexpr (SHAW) {
        // in the band: each group of 8 keys reads its 8 relative logits from
        // one base (the row padding keeps it in the row; end labels come from
        // registers)
        float rlv[16], rvv[16];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int d0 = kofs + 16 * g;
          const int bidx = min(max(d0 - dlo, -PADL), lay.lrs - PADL - SPAN);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            rlv[8 * g + e] = HAS_WK ? RG[bidx + KSTR * e] : 0.f;
            rvv[8 * g + e] = HAS_WV ? RV[bidx + KSTR * e] : 0.f;
          }
        }
        float gs = 0.f, ws = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ko = 16 * (i >> 3) + KSTR * (i & 7);
          const int delta = kofs + ko;
          const bool lo = delta <= -band, hi = delta >= hi_from;
          const float rl = lo ? rl_lo : (hi ? rl_hi : rlv[i]);
          const float rv = lo ? rv_lo : (hi ? rv_hi : rvv[i]);
          const bool vis = ko <= lim;
          const float pv = vis ? fast_exp2(fmaf(s[i], p.scale_log2, rl) - lse2) : 0.f;
          pw[i] = pv;
          ds[i] = vis ? pv * (dp[i] + rv - dd) : 0.f;
          gs += ds[i];
          ws += pv;
        }
        g_all += gs;
        w_all += ws;
        if (!p.causal) {
          // keys at the upper end label (none is visible under the causal mask)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const bool hi = kofs + 16 * (i >> 3) + KSTR * (i & 7) >= hi_from;
            g_hi += hi ? ds[i] : 0.f;
            w_hi += hi ? pw[i] : 0.f;
          }
        }
        // a group that holds a reachable in-band label is stored whole at its
        // own entries (entries of other labels are rewritten in the epilogue;
        // the padding absorbs the rest): every such label holds exactly this
        // one key of the row
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int d0 = kofs + 16 * g;
          if (q_ok && d0 + (SPAN - 1) >= wb_lo && d0 <= wb_hi) {
            const int base = d0 - dlo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if constexpr (HAS_WK) RG[base + KSTR * e] = ds[8 * g + e];
              if constexpr (HAS_WV) RV[base + KSTR * e] = pw[8 * g + e];
            }
          }
        }
      } else if constexpr (GRID) {
        // 2-D window: each pair's entry of the head's table, from the (dy, dx)
        // of key minus query (token t at row t div M, taken in fp32 as
        // (t + 1/2) / M, exact for t < 2^22, and column t mod M); keys and rows
        // past n read a clamped entry and weigh 0
        const int M = p.grid_m;
        const int qc = min(qi, p.n - 1);
        const int yq = (int)(((float)qc + 0.5f) * p.grid_inv), xq = qc - yq * M;
        int ent[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ko = 16 * (i >> 3) + KSTR * (i & 7);
          const int j = min(jb + hoff + ko, p.n - 1);
          const int yj = (int)(((float)j + 0.5f) * p.grid_inv), xj = j - yj * M;
          ent[i] = (yj - yq + M - 1) * (2 * M - 1) + (xj - xq + M - 1);
          const bool vis = ko <= lim;
          // the exponential for every lane, then a select
          float ex = fast_exp2(fmaf(s[i], p.scale_log2, TB[ent[i]]) - lse2);
          asm volatile("" : "+v"(ex));
          const float pv = vis ? ex : 0.f;
          pw[i] = pv;
          ds[i] = vis ? pv * (dp[i] - dd) : 0.f;
        }
        // each register's 32 lanes of a half hold distinct entries (rows past
        // n, which share the clamped row's entries, add nothing); the
        // registers follow one another in program order
        if (want_db && q_ok) {
#pragma unroll
          for (int i = 0; i < 16; ++i) GB[ent[i]] += ds[i];
        }
      } else if constexpr (LAB) {
        // edge labels: the 32 keys of the block lie in two 16-byte chunks of
        // the query's label row; this lane's keys are bytes hoff + KSTR e of
        // each.  Chunks past the row's readable length (keys past n, which
        // weigh 0) re-read its last chunk; rows past n read row n - 1.
        const uint8_t* lrow = labg + (int64_t)min(qi, p.n - 1) * p.lab_sn;
        const int cmax = ((p.n + 15) & ~15) - 16;
        uint4 ch[2];
#pragma unroll
        for (int g = 0; g < 2; ++g)
          ch[g] = *reinterpret_cast<const uint4*>(lrow + min(jb + 16 * g, cmax));
        int ent[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint4 c4 = ch[i >> 3];
          const int e = i & 7;
          uint32_t lb;
          if constexpr (BF16) {
            // bytes 8 hh + e: word (e >> 2) of the lane's 8-byte half
            const uint32_t w = (e >> 2) ? (hh ? c4.w : c4.y) : (hh ? c4.z : c4.x);
            lb = (w >> (8 * (e & 3))) & 0xffu;
          } else {
            // bytes hh + 2 e: word e >> 1, byte 2 (e & 1) + hh
            const uint32_t w = (e >> 1) == 0 ? c4.x : (e >> 1) == 1 ? c4.y
                             : (e >> 1) == 2 ? c4.z : c4.w;
            lb = (w >> (8 * (2 * (e & 1) + hh))) & 0xffu;
          }
          ent[i] = min((int)lb, p.t5.nb - 1);  // a label past the table reads its last entry
          const int ko = 16 * (i >> 3) + KSTR * (i & 7);
          const bool vis = ko <= lim;
          float ex = fast_exp2(fmaf(s[i], p.scale_log2, TB[ent[i]]) - lse2);
          asm volatile("" : "+v"(ex));
          const float pv = vis ? ex : 0.f;
          pw[i] = pv;
          ds[i] = vis ? pv * (dp[i] - dd) : 0.f;
        }
        // one row per query and lane half: a single writer
        if (want_db) {
#pragma unroll
          for (int i = 0; i < 16; ++i) GB[ent[i]] += ds[i];
        }
      } else {
        // T5 in the band: the bias of each key's bucket
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ko = 16 * (i >> 3) + KSTR * (i & 7);
          const int delta = kofs + ko;
          float rl = 0.f;
          if constexpr (T5) rl = TB[min(max(delta, -dist), dist) + dist];
          const bool vis = ko <= lim;
          const float pv = vis ? fast_exp2(fmaf(s[i], p.scale_log2, rl) - lse2) : 0.f;
          pw[i] = pv;
          ds[i] = vis ? pv * (dp[i] - dd) : 0.f;
        }
        if constexpr (T5) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int delta = kofs + 16 * (i >> 3) + KSTR * (i & 7);
            if (delta <= -band) {
              g_lo += ds[i];
            } else if (delta >= hi_from) {
              g_hi += ds[i];
            } else if (want_db && q_ok && qi + delta < p.n) {
              GB[TBI[delta + dist]] += ds[i];
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
  block_sync();  // the ring is free
  // the Q and dZ tiles for the partial table gradients, rebuilt in the ring
  // from the row fragments each lane holds (same layout as a DMA'd tile)
  if constexpr (ROWS) {
    if constexpr (XL) {
      // the table gradient takes q + v: the row and v again (the lane's q
      // fragments hold q + u by now)
      Op qq[NKS];
      load_row_frags<BF16, D>(qg + (int64_t)qr * p.q_sn, hh, qq);
      load_row_frags<BF16, D>(reinterpret_cast<const T*>(p.xl_v) + h * p.xl_v_sh, hh, xv);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qop[ks] = op_add(qq[ks], xv[ks]);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (BF16) {
        const int o = tile_offset<ROWB>(qrow, (2 * ks + hh) * 16);
        if constexpr (HAS_WK) *reinterpret_cast<bf16x8*>(smem + o) = qop[ks];
        if constexpr (HAS_WV) *reinterpret_cast<bf16x8*>(smem + BR * ROWB + o) = zop[ks];
      } else {
        const int o = tile_offset<ROWB>(qrow, (2 * ks + hh) * 4);
        if constexpr (HAS_WK) *reinterpret_cast<float*>(smem + o) = qop[ks];
        if constexpr (HAS_WV) *reinterpret_cast<float*>(smem + BR * ROWB + o) = zop[ks];
      }
    }
  }

  // ---- epilogue: final label sums of this row.  In-band labels hold their
  // key's dS (and P) where the pair is visible, zero elsewhere; the lower end
  // label takes what the row's total leaves after the in-band and upper sums.
  // Tables by edge label: the two lane halves' sums of each label, added.
  if constexpr (GRAPH) {
    compiler_fence();
    const float* g0 = reinterpret_cast<const float*>(smem + lay.gb) + 2 * qrow * lay.gbs;
    const float* w0 = reinterpret_cast<const float*>(smem + lay.gw) + 2 * qrow * lay.gbs;
    for (int x = hh; x < p.nr; x += 2) {
      if constexpr (HAS_WK) RG[x] = q_ok ? g0[x] + g0[lay.gbs + x] : 0.f;
      if constexpr (HAS_WV) RV[x] = q_ok ? w0[x] + w0[lay.gbs + x] : 0.f;
    }
    compiler_fence();  // the other half of this wave wrote the rest of the row
  } else if constexpr (ROWS) {
    const float gall = halves_sum(g_all), wall = halves_sum(w_all);
    const float gh = halves_sum(g_hi), wh = halves_sum(w_hi);
    const int x_lo = -p.r_lo;         // label -c (present when r_lo == 0)
    const int x_hi = 2 * c - p.r_lo;  // label +c (present when < nr)
    float gin = 0.f, win = 0.f;
    for (int x = hh; x < p.nr; x += 2) {
      if (x == x_lo || x == x_hi) continue;
      const int delta = x + p.r_lo - c;
      const int j = qi + delta;
      const bool vis = q_ok && j >= 0 && j < kv_len && (!p.causal || delta <= 0);
      if constexpr (HAS_WK) {
        const float v = vis ? RG[x] : 0.f;
        RG[x] = v;
        gin += v;
      }
      if constexpr (HAS_WV) {
        const float v = vis ? RV[x] : 0.f;
        RV[x] = v;
        win += v;
      }
    }
    gin = halves_sum(gin);
    win = halves_sum(win);
    const float gl = gall - gin - gh, wl = wall - win - wh;
    if (hh == 0) {
      if (x_lo == 0) {
        if constexpr (HAS_WK) RG[0] = q_ok ? gl + (x_hi == 0 ? gh : 0.f) : 0.f;
        if constexpr (HAS_WV) RV[0] = q_ok ? wl + (x_hi == 0 ? wh : 0.f) : 0.f;
      }
      if (x_hi != x_lo && x_hi < p.nr) {
        if constexpr (HAS_WK) RG[x_hi] = q_ok ? gh : 0.f;
        if constexpr (HAS_WV) RV[x_hi] = q_ok ? wh : 0.f;
      }
    }
    compiler_fence();  // the other half of this wave wrote the rest of the row
  }

  // ---- dQ^T += (w^K)^T G^T with the resident w^K rows (Transformer-XL: into
  // an accumulator of its own first, so that the tile's sums over its rows of
  // the content part, s sum dS k (-> du), and of this part, s sum G R (-> dv),
  // can be taken apart)
  [[maybe_unused]] f32x16 gw[DVB];
  if constexpr (XL) {
#pragma unroll
    for (int mb = 0; mb < DVB; ++mb) gw[mb] = f32x16{};
  }
  auto add_table_part = [&](f32x16 (&acc)[DVB]) __attribute__((always_inline)) {
    const int nls = (p.nr + 15) / 16;
    const uint32_t tk_lds = smem_addr + (uint32_t)lay.tk;
    for (int ls = 0; ls < nls; ++ls) {
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
          frag_col_issue<ROWB, D>(tk_lds, ls * 16, 32 * mb, lane, wlo[mb], whi[mb]);
        frag_col_wait(wlo, whi);
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb) acc[mb] = mfma(frag_join(wlo[mb], whi[mb]), bw, acc[mb]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int x = ls * 16 + 2 * e + hh;
          const float w = x < p.nr ? RG[x] : 0.f;
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) {
            const int dcol = min(32 * mb + ql, D - 1);
            acc[mb] = mfma(elem_f32<ROWB>(smem + lay.tk, ls * 16 + 2 * e + hh, dcol), w, acc[mb]);
          }
        }
      }
    }
  };
  if constexpr (XL) {
    add_table_part(gw);
    if (p.ws_pu) {
      // this tile's sums over its rows: the content part, then the table part
      const int64_t tile_id = (int64_t)bh * p.n_qtiles + qt;
      float* xs = reinterpret_cast<float*>(smem + lay.xs);
      float* dst = p.ws_pu + tile_id * 2 * D;
      auto rows_sum = [&](const f32x16 (&acc)[DVB], float* out) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            // the 32 lanes of a half hold the same d and 32 queries
            float v = acc[mb][i];
#pragma unroll
            for (int m = 16; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
            const int dd = 32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3);
            if (ql == 0 && dd < D) xs[wave * D + dd] = v;
          }
        block_sync();
        for (int dd = tid; dd < D; dd += NT) {
          float sum = 0.f;
          for (int w = 0; w < NW; ++w) sum += xs[w * D + dd];
          out[dd] = sum;
        }
        block_sync();
      };
      rows_sum(dq, dst);
      rows_sum(gw, dst + D);
    }
#pragma unroll
    for (int mb = 0; mb < DVB; ++mb) dq[mb] += gw[mb];
  } else if constexpr (SHAW && HAS_WK) {
    add_table_part(dq);
  }
  if (q_ok) store_row_block<T, D>(dqg + (int64_t)qi * p.dq_sn, dq, p.scale, hh);

  // ---- partial table gradients of this tile: (w^K)' = s Q^T G, (w^V)' = dZ^T W
  if constexpr (ROWS) {
    block_sync();  // the Q and dZ tiles are written; every row is final
    const int nlb = (p.nr + 31) / 32;
    const int per = nlb * DVB;
    constexpr int NWHICH = (HAS_WK ? 1 : 0) + (HAS_WV ? 1 : 0);
    const int64_t tile_id = (int64_t)bh * p.n_qtiles + qt;
    for (int tt = wave; tt < per * NWHICH; tt += NW) {
      const bool isv = HAS_WK ? tt >= per : true;
      const int r = (HAS_WK && isv) ? tt - per : tt;
      const int lb = r / DVB, mb = r - lb * DVB;
      const float* Gr = reinterpret_cast<const float*>(smem + (isv ? lay.rv : lay.rg)) + PADL;
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
  if constexpr (GRID || LAB) {
    if (want_db) {
      block_sync();
      const float* gb0 = reinterpret_cast<const float*>(smem + lay.gb);
      const int64_t tile_id = (int64_t)bh * p.n_qtiles + qt;
      for (int e = tid; e < p.t5.nb; e += NT) {
        float acc = 0.f;
        for (int slot = 0; slot < (GRID ? 2 * NW : 2 * BR); ++slot) acc += gb0[slot * lay.gbs + e];
        p.ws_pb[tile_id * p.t5.nb + e] = acc;
      }
    }
  }
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
// Table and bias gradients: sums of the per-tile partials in a fixed order,
// done by the dk/dv workgroups after their keys.  Role ids: first one
// workgroup per (table head, label) of d w^K, then of d w^V, then the bias
// gradient's workgroups (nt entries each).
// ---------------------------------------------------------------------------
// table rows per head: 2 clip + 1 labels by clipped offset, NL by edge label
__host__ __device__ inline int table_labels(const BwdParams& p) {
  return p.nlab ? p.nlab : 2 * p.clip + 1;
}
__host__ __device__ inline int reduce_tables_rows(const BwdParams& p, int which) {
  const int ht = which ? (p.dwv ? p.htv : 0) : (p.dwk ? p.htk : 0);
  return ht * table_labels(p);
}
// Groups of threads that share one bias-gradient entry: enough for about 16
// partials each (a power of two up to the workgroup).
__host__ __device__ inline int bias_groups(const BwdParams& p, int nt) {
  const int64_t U = (int64_t)p.B * ((p.ob && p.hb == 1) ? p.H : 1) * p.n_qtiles;
  int G = 1;
  while (G < nt && (int64_t)G * 16 < U) G *= 2;
  return G;
}
// (Transformer-XL's du and dv rows only in that mode's kernels: read in the
// others, their fields would hold registers through the whole kernel)
template <bool XL>
__host__ __device__ inline int reduce_xl_rows(const BwdParams& p) {
  if constexpr (XL) return (p.du ? p.hu : 0) + (p.dvb ? p.hv : 0);
  return 0;
}
template <bool XL>
__host__ __device__ inline int reduce_role_count(const BwdParams& p, int nt) {
  int n = reduce_tables_rows(p, 0) + reduce_tables_rows(p, 1) + reduce_xl_rows<XL>(p);
  if (p.db) {
    const int64_t total = p.ob ? (int64_t)p.hb * p.ob_n : (int64_t)p.t5.nb * p.H;
    const int epr = nt / bias_groups(p, nt);
    n += (int)((total + epr - 1) / epr);
  }
  return n;
}

// One (table head, label) row of d w^K or d w^V: the nt threads form nt/d
// groups of d columns; group g sums terms g, g + G, ... and the groups are
// added in order.
__device__ void reduce_table_row(const BwdParams& p, int which, int row, int nt) {
  float* out = which ? p.dwv : p.dwk;
  const int ht = which ? p.htv : p.htk;
  const int nlab = table_labels(p);
  const int hq = row / nlab, r = row - hq * nlab;
  const int d = p.d, G = nt / d;
  const int tid = threadIdx.x;
  const int dd = tid % d, g = tid / d;
  const int x = r - p.r_lo;
  float acc = 0.f;
  if (x >= 0 && x < p.nr) {
    const float* part = which ? p.ws_pv : p.ws_pk;
    const int h_lo = ht == 1 ? 0 : hq, hn = ht == 1 ? p.H : 1;
    const int nq = p.n_qtiles;
    const int U = p.B * hn * nq;  // term u: (b, head, query tile)
    auto term = [&](int u) __attribute__((always_inline)) {
      const int tq = u % nq, bh2 = u / nq;
      const int b = bh2 / hn, hh = h_lo + (bh2 - b * hn);
      return part[(((int64_t)(b * p.H + hh) * nq + tq) * p.nr + x) * d + dd];
    };
    // eight loads in flight, then added in order
    int u = g;
    for (; u + 7 * G < U; u += 8 * G) {
      float t8[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t8[k] = term(u + k * G);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += t8[k];
    }
    for (; u < U; u += G) acc += term(u);
  }
  extern __shared__ __align__(16) unsigned char smem[];
  float* red = reinterpret_cast<float*>(smem);
  red[tid] = acc;
  __syncthreads();
  if (g == 0) {
    float sum = 0.f;
    for (int k = 0; k < G; ++k) sum += red[k * d + dd];
    const int64_t sh = which ? p.dwv_sh : p.dwk_sh, sr = which ? p.dwv_sr : p.dwk_sr;
    out[hq * sh + r * sr + dd] = sum;
  }
}

// Bias gradient entries [blk * nt, blk * nt + nt): one thread each.
__device__ void reduce_bias(const BwdParams& p, int blk, int nt) {
  // G groups of EPR threads: thread (g, el) sums terms g, g + G, ... of entry
  // blk * EPR + el, and the groups are added in order
  const int G = bias_groups(p, nt), EPR = nt / G;
  const int tid = threadIdx.x, g = tid / EPR, el = tid - g * EPR;
  const int64_t idx = (int64_t)blk * EPR + el;
  const int nq = p.n_qtiles;
  const int nbt = p.t5.nb;  // entries per head in the partials
  const bool ob = p.ob != 0;
  const int nw = p.ob_n;
  const int64_t total = ob ? (int64_t)p.hb * nw : (int64_t)nbt * p.H;
  const bool live = idx < total;
  // scalar-bias table [hb, ob_n] (entries outside the loaded window, offsets
  // no pair reaches, get zero) or T5 table [nb, H]
  int hq = 0, w = 0, e = -1;
  if (live) {
    if (ob) {
      w = (int)(idx % nw);
      hq = (int)(idx / nw);
      e = w - p.ob_lo;
      if (e >= nbt) e = -1;
    } else {
      hq = (int)(idx % p.H);
      e = (int)(idx / p.H);
    }
  }
  const int hn = (ob && p.hb == 1) ? p.H : 1, h_lo = hn == 1 ? hq : 0;
  float acc = 0.f;
  if (live && e >= 0) {
    const int64_t U = (int64_t)p.B * hn * nq;  // term u: (b, head, query tile)
    auto term = [&](int64_t u) __attribute__((always_inline)) {
      const int t = (int)(u % nq);
      const int bh2 = (int)(u / nq);
      const int b = bh2 / hn, hh = h_lo + (bh2 - b * hn);
      return p.ws_pb[((int64_t)(b * p.H + hh) * nq + t) * nbt + e];
    };
    int64_t u = g;
    for (; u + 7 * G < U; u += 8 * G) {
      float t8[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t8[k] = term(u + k * G);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += t8[k];
    }
    for (; u < U; u += G) acc += term(u);
  }
  extern __shared__ __align__(16) unsigned char smem[];
  float* red = reinterpret_cast<float*>(smem);
  red[tid] = acc;
  __syncthreads();
  if (g == 0 && live) {
    float sum = 0.f;
    for (int k = 0; k < G; ++k) sum += red[k * EPR + el];
    if (ob) p.db[hq * p.db_s0 + w * p.db_s1] = sum;
    else p.db[e * p.db_s0 + hq * p.db_s1] = sum;
  }
}

// Transformer-XL: one head row of du (which = 0) or dv (which = 1), s times
// the sum of the query tiles' partials over the batch (and over the heads
// for one shared vector); the nt threads form nt/d groups of d columns, added
// in order as for the tables.
__device__ void reduce_xl_row(const BwdParams& p, int which, int hq, int nt) {
  const int hx = which ? p.hv : p.hu;
  const int d = p.d, G = nt / d;
  const int tid = threadIdx.x;
  const int dd = tid % d, g = tid / d;
  const int h_lo = hx == 1 ? 0 : hq, hn = hx == 1 ? p.H : 1;
  const int nq = p.n_qtiles;
  const int U = p.B * hn * nq;  // term u: (b, head, query tile)
  float acc = 0.f;
  if (g < G) {
    auto term = [&](int u) __attribute__((always_inline)) {
      const int tq = u % nq, bh2 = u / nq;
      const int b = bh2 / hn, hh = h_lo + (bh2 - b * hn);
      return p.ws_pu[(((int64_t)(b * p.H + hh) * nq + tq) * 2 + which) * d + dd];
    };
    int u = g;
    for (; u + 7 * G < U; u += 8 * G) {
      float t8[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t8[k] = term(u + k * G);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += t8[k];
    }
    for (; u < U; u += G) acc += term(u);
  }
  extern __shared__ __align__(16) unsigned char smem[];
  float* red = reinterpret_cast<float*>(smem);
  red[tid] = acc;
  __syncthreads();
  if (g == 0) {
    float sum = 0.f;
    for (int k = 0; k < G; ++k) sum += red[k * d + dd];
    if (which) p.dvb[hq * p.dvb_sh + dd] = sum * p.scale;
    else p.du[hq * p.du_sh + dd] = sum * p.scale;
  }
}

template <bool XL>
__device__ void reduce_role(const BwdParams& p, int role, int nt) {
  const int rk = reduce_tables_rows(p, 0), rv = reduce_tables_rows(p, 1);
  const int ru = XL ? (p.du ? p.hu : 0) : 0, rx = reduce_xl_rows<XL>(p);
  if (role < rk) {
    reduce_table_row(p, 0, role, nt);
  } else if (role < rk + rv) {
    reduce_table_row(p, 1, role - rk, nt);
  } else if (XL && role < rk + rv + rx) {
    const int r = role - rk - rv;
    if (r < ru) reduce_xl_row(p, 0, r, nt);
    else reduce_xl_row(p, 1, r - ru, nt);
  } else {
    reduce_bias(p, role - rk - rv - rx, nt);
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
  // Transformer-XL runs the key-table path with R as the table; the tables
  // by edge label (GRAPH) run it with each pair's label as its table row
  constexpr bool XL = MODE == kRelXL, GRAPH = MODE == kRelGraph;
  constexpr bool SHAW = MODE == kRelShaw || XL || GRAPH, T5 = MODE == kRelT5;
  constexpr bool GRID = MODE == kRelGrid, LAB = MODE == kRelLabel;
  constexpr bool ROWS = SHAW && (HAS_WK || HAS_WV);

  const int n_kv = p.B * p.H * p.n_ktiles;
  const int lid = xcd_remap(blockIdx.x, n_kv);
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
  const int r_hi = p.r_lo + p.nr - 1;

  const LayKV lay = make_lay_kv<BF16, D, NW, BQ>(MODE, HAS_WK, HAS_WV, p.nr, dist, p.t5.nb);
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char RELATTN_LDS* smem_lds = (unsigned char RELATTN_LDS*)smem;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem_lds;
  float* TB = reinterpret_cast<float*>(smem + lay.tb);
  float* RLt = reinterpret_cast<float*>(smem + lay.rl);
  float* RVt = reinterpret_cast<float*>(smem + lay.rv);
  float* TAIL = reinterpret_cast<float*>(smem + lay.tail);  // [a_lo | a_hi | b_lo | b_hi][BQ]
  float* XB = reinterpret_cast<float*>(smem + lay.xb);

  const T* qg = reinterpret_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const T* kg = reinterpret_cast<const T*>(p.k) + b * p.k_sb + h * p.k_sh;
  const T* vg = reinterpret_cast<const T*>(p.v) + b * p.v_sb + h * p.v_sh;
  const T* zg = reinterpret_cast<const T*>(p.dout) + b * p.do_sb + h * p.do_sh;
  T* dkg = reinterpret_cast<T*>(p.dk) + b * p.dk_sb + h * p.dk_sh;
  T* dvg = reinterpret_cast<T*>(p.dv) + b * p.dv_sb + h * p.dv_sh;
  const float* stat = p.ws_stat + (int64_t)bh * 2 * p.n_pad;

  // ---- requested at once: this lane's k and v row (B operands, straight
  // from memory), the table rows of the reachable labels (LDS, resident) or
  // the bias window, and the first query tile
  int kv_len = p.n;
  if (p.key_lens) kv_len = min(max(p.key_lens[b], 0), p.n);
  // query tiles that can see a key of this workgroup
  const int t_lo = p.causal ? k0 / BQ : 0;
  const int t_end = (k0 < kv_len) ? (p.n + BQ - 1) / BQ : t_lo;
  const int kr = min(kj, p.n - 1);
  Op kop[NKS], vop[NKS];
  load_row_frags<BF16, D>(kg + (int64_t)kr * p.k_sn, hh, kop);
  load_row_frags<BF16, D>(vg + (int64_t)kr * p.v_sn, hh, vop);
  // Transformer-XL: the content logit's term u . k_j of this lane's key (log2
  // units), and its running sum of dS for dk's share s u sum_i dS_ij
  [[maybe_unused]] float ukl2 = 0.f, cs = 0.f;
  if constexpr (XL) {
    Op xu[NKS];
    load_row_frags<BF16, D>(reinterpret_cast<const T*>(p.xl_u) + h * p.xl_u_sh, hh, xu);
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (BF16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf((float)xu[ks][e], (float)kop[ks][e], part);
      } else {
        part = fmaf(xu[ks], kop[ks], part);
      }
    }
    ukl2 = halves_sum(part) * p.scale_log2;
  }
  if constexpr (T5) {
    for (int x = tid; x <= 2 * dist; x += NT) {
      const int entry = p.ob ? x : t5_bucket(x - dist, p.t5);
      TB[x] = kLog2e * p.t5_bias[(entry + p.ob_lo) * p.tb_sb + h * p.tb_sh];
    }
  }
  if constexpr (GRID || LAB) {
    for (int x = tid; x < p.t5.nb; x += NT) TB[x] = kLog2e * p.t5_bias[x * p.tb_sb + h * p.tb_sh];
  }
  compiler_fence();
  if constexpr (SHAW && HAS_WK)
    dma_tile<ROWB, NW>(smem_lds + lay.tk, reinterpret_cast<const T*>(p.wk) + h * p.wk_sh,
                       p.wk_sr, p.r_lo, r_hi, lay.tab_rows, wave, lane);
  if constexpr (SHAW && HAS_WV)
    dma_tile<ROWB, NW>(smem_lds + lay.tv, reinterpret_cast<const T*>(p.wv) + h * p.wv_sh,
                       p.wv_sr, p.r_lo, r_hi, lay.tab_rows, wave, lane);
  auto issue = [&](int t, int stage) __attribute__((always_inline)) {
    unsigned char RELATTN_LDS* st = smem_lds + stage * lay.stage;
    const int q0 = t * BQ;
    stage_pair<ROWB, NW, BQ>(st + lay.q, qg, p.q_sn, zg, p.do_sn, q0, p.n - 1, wave, lane);
    if (wave == 0) {
      dma_flat<1, 4>(st + lay.lse, stat + q0, 256, 0, lane);
      dma_flat<1, 4>(st + lay.dd, stat + p.n_pad + q0, 256, 0, lane);
    }
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
  // |delta| >= band: an end label (none in the 2-D window or by edge label)
  const int band = T5 ? dist : ((GRID || LAB || GRAPH) ? (1 << 30) : c);
  const int hi_from = max(band, 1 - band);  // delta >= hi_from: the upper end
  // 2-D window: this lane's key on the M x M grid (row (t + 1/2) / M in fp32,
  // exact for t < 2^22)
  [[maybe_unused]] int yk = 0, xk = 0;
  if constexpr (GRID) {
    const int kc = min(kj, p.n - 1);
    yk = (int)(((float)kc + 0.5f) * p.grid_inv);
    xk = kc - yk * p.grid_m;
  }
  // edge labels: this lane's key column of the batch entry's label matrix
  // (keys past n read column n - 1; they are stored as zeros)
  [[maybe_unused]] const uint8_t* labk =
      (LAB || GRAPH) ? p.lab + b * p.lab_sb + min(kj, p.n - 1) : nullptr;

  // 16 per-query values of this lane's registers: vector reads of 4
  // consecutive queries (bf16 register order), else one by one
  auto per_query = [&](const float* arr, int qb, float (&out)[16]) __attribute__((always_inline)) {
    if constexpr (BF16) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(arr + 32 * qb + hoff + 16 * g + 4 * hv);
#pragma unroll
          for (int e = 0; e < 4; ++e) out[8 * g + 4 * hv + e] = a[e];
        }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) out[i] = arr[32 * qb + hoff + 16 * (i >> 3) + KSTR * (i & 7)];
    }
  };

  for (int t = t_lo; t < t_end; ++t) {
    const int stg = (t - t_lo) & 1;
    wait_vm<0>();
    block_sync();  // tile t (and the tables) landed everywhere; the other stage
                   // and the rows are free
    const unsigned char* S0 = smem + stg * lay.stage;
    const unsigned char* Qt = S0 + lay.q;
    const unsigned char* Zt = S0 + lay.z;
    const float* LS = reinterpret_cast<const float*>(S0 + lay.lse);
    const float* DD = reinterpret_cast<const float*>(S0 + lay.dd);
    const int q0 = t * BQ;

    if constexpr (XL) {
      if (t == t_lo) {
        // v . R_r for every resident table row (landed with the first tile)
        const T* vbp = reinterpret_cast<const T*>(p.xl_v) + h * p.xl_v_sh;
        const unsigned char* tk = smem + lay.tk;
        for (int x = tid; x < lay.tab_rows; x += NT) {
          float acc = 0.f;
          for (int dd = 0; dd < D; ++dd)
            acc = fmaf((float)vbp[dd],
                       (float)*reinterpret_cast<const T*>(tk + tile_offset<ROWB>(x, dd * G::ESZ)),
                       acc);
          XB[x] = acc;
        }
        block_sync();
      }
    }
    if constexpr (ROWS) {
      // relative rows of the tile's queries: C[label, query] = w_r . x_q with
      // x = q (key table, scaled to log2 units) or dz (value table), and the
      // two end labels less lse (key table) or D (value table)
      constexpr int NWHICH = (HAS_WK ? 1 : 0) + (HAS_WV ? 1 : 0);
      const int nlb = lay.tab_rows / 32;
      for (int it = wave; it < NQB * nlb * NWHICH; it += NW) {
        const int which = it % NWHICH, rest = it / NWHICH;
        const int lb = rest % nlb, qb = rest / nlb;
        const bool isv = HAS_WK ? which == 1 : true;
        const unsigned char* tab = smem + (isv ? lay.tv : lay.tk);
        const unsigned char* X = isv ? Zt : Qt;
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if constexpr (BF16) {
            acc = mfma(frag_row<ROWB>(tab, lb * 32 + ql, 2 * ks + hh),
                       frag_row<ROWB>(X, 32 * qb + ql, 2 * ks + hh), acc);
          } else {
            acc = mfma(elem_f32<ROWB>(tab, lb * 32 + ql, 2 * ks + hh),
                       elem_f32<ROWB>(X, 32 * qb + ql, 2 * ks + hh), acc);
          }
        }
        const int lq = 32 * qb + ql;
        float* row = (isv ? RVt : RLt) + lq * lay.lrs;
        const float mul = isv ? 1.f : p.scale_log2;
        const float sub = isv ? DD[lq] : LS[lq];
        float* tl = TAIL + (isv ? 2 * BQ : 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int x = lb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          // Transformer-XL: (q + v) . R_r = q . R_r + v . R_r
          const float v = (XL ? acc[i] + XB[x] : acc[i]) * mul;
          if (x < p.nr) row[x] = v;
          if (x == 0) tl[lq] = v - sub;
          if (x == p.nr - 1) tl[BQ + lq] = v - sub;
        }
      }
      block_sync();
    }
    // the next tile, requested once this tile's rows are in place
    if (t + 1 < t_end) issue(t + 1, stg ^ 1);
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
      // offsets delta = key - query of the block: all at one end label (or no
      // relative term)?  Keys past the key length are not masked here: their
      // columns are independent and are written as zeros.
      const bool all_lo = (wk0 + 31) - qb0 <= -band;
      const bool all_hi = wk0 - (qb0 + 31) >= hi_from;
      const bool off_band = MODE == kRelNone || all_lo || all_hi;
      // some query of the block past n, or before some key of the wave
      const bool need_mask = qb0 + 31 >= p.n || (p.causal && wk0 + 31 > qb0);
      float pw[16], ds[16];
      if (off_band) {
        // per query: the end label's relative logit less lse, and its value
        // term less D
        float av[16], bv[16];
        if constexpr (ROWS && HAS_WK) {
          per_query(TAIL + (all_hi ? BQ : 0), qb, av);
        } else {
          per_query(LS, qb, av);
          const float e = T5 ? (all_hi ? TB[2 * dist] : TB[0]) : 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) av[i] = e - av[i];
        }
        if constexpr (ROWS && HAS_WV) {
          per_query(TAIL + 2 * BQ + (all_hi ? BQ : 0), qb, bv);
        } else {
          per_query(DD, qb, bv);
#pragma unroll
          for (int i = 0; i < 16; ++i) bv[i] = -bv[i];
        }
        auto run = [&](auto mask_tag) __attribute__((always_inline)) {
          constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float pv = fast_exp2(fmaf(s[i], p.scale_log2, XL ? av[i] + ukl2 : av[i]));
            if constexpr (MASK) {
              const int qq = qb0 + hoff + 16 * (i >> 3) + KSTR * (i & 7);
              pv = (qq < p.n && (!p.causal || kj <= qq)) ? pv : 0.f;
            }
            pw[i] = pv;
            ds[i] = pv * (dp[i] + bv[i]);
          }
        };
        if (need_mask) {
          run(std::true_type{});
        } else {
          run(std::false_type{});
        }
      } else {
        float lsv[16], ddv[16];
        per_query(LS, qb, lsv);
        per_query(DD, qb, ddv);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int lq = 32 * qb + hoff + 16 * (i >> 3) + KSTR * (i & 7);
          const int qq = q0 + lq;
          const int delta = kj - qq;
          float rl = 0.f, rv = 0.f;
          if constexpr (SHAW) {
            // the pair's table row: its clipped offset, or its edge label
            const int x = GRAPH ? min((int)labk[(int64_t)min(qq, p.n - 1) * p.lab_sn], p.nr - 1)
                                : min(max(delta + c - p.r_lo, 0), p.nr - 1);
            if constexpr (HAS_WK) rl = RLt[lq * lay.lrs + x];
            if constexpr (HAS_WV) rv = RVt[lq * lay.lrs + x];
          } else if constexpr (T5) {
            rl = TB[min(max(delta, -dist), dist) + dist];
          } else if constexpr (GRID) {
            const int M = p.grid_m;
            const int qc = min(qq, p.n - 1);
            const int yq = (int)(((float)qc + 0.5f) * p.grid_inv), xq = qc - yq * M;
            rl = TB[(yk - yq + M - 1) * (2 * M - 1) + (xk - xq + M - 1)];
          } else if constexpr (LAB) {
            const int lb = labk[(int64_t)min(qq, p.n - 1) * p.lab_sn];
            rl = TB[min(lb, p.t5.nb - 1)];
          }
          const bool vis = qq < p.n && (!p.causal || delta <= 0);
          // the exponential for every lane, then a select (a conditional
          // exponential becomes a branch per element, each waiting for its
          // own row reads)
          float ex = fast_exp2(fmaf(s[i], p.scale_log2, XL ? rl + ukl2 : rl) - lsv[i]);
          asm volatile("" : "+v"(ex));
          const float pv = vis ? ex : 0.f;
          pw[i] = pv;
          ds[i] = vis ? pv * (dp[i] + rv - ddv[i]) : 0.f;
        }
      }
      if constexpr (XL) {
#pragma unroll
        for (int i = 0; i < 16; ++i) cs += ds[i];
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
  if constexpr (XL) {
    // dk_j = s sum_i dS_ij (q_i + u): add u times the key's sum of dS
    const float cst = halves_sum(cs);
    const T* up = reinterpret_cast<const T*>(p.xl_u) + h * p.xl_u_sh;
#pragma unroll
    for (int mb = 0; mb < DVB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int dd = 32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (dd < D) dk[mb][i] = fmaf((float)up[dd], cst, dk[mb][i]);
      }
  }
  if (kj < p.n) {
    // a key past the key length is seen by no query: its gradients are zero
    store_row_block<T, D>(dkg + (int64_t)kj * p.dk_sn, dk, p.scale, hh, !k_ok);
    store_row_block<T, D>(dvg + (int64_t)kj * p.dv_sn, dv, 1.f, hh, !k_ok);
  }

  // Then the table and bias gradients: sums of the partials the dq kernel
  // (launched before on the same stream) wrote.  Under the causal mask the
  // last key tiles of a head see the fewest queries and finish first; they
  // take every reduction role.  Otherwise all workgroups share them.
  const int n_roles = reduce_role_count<XL>(p, NT);
  if (n_roles > 0) {
    const int BH = p.B * p.H;
    int first, stride;
    if (p.causal && p.n_ktiles > 1) {
      const int light = (p.n_ktiles + 1) / 2;  // key tiles kt >= n_ktiles - light
      if (kt < p.n_ktiles - light) return;
      first = (kt - (p.n_ktiles - light)) * BH + bh;
      stride = light * BH;
    } else {
      first = lid;
      stride = n_kv;
    }
    for (int role = first; role < n_roles; role += stride) {
      block_sync();  // the LDS the role uses is free
      reduce_role<XL>(p, role, NT);
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
  // the tiny dq shape of the key-table modes (bf16, d <= 64): one wave,
  // 32-key tiles
  static constexpr int QW_TINY = 1;
  static constexpr int QBC_TINY = 32;
};

template <bool BF16, int D>
static size_t lds_q_t(int qwaves, RelMode mode, bool has_wk, bool has_wv, int nr, int t5_dist,
                      int nb, bool want_db) {
  using S = BwdShape<BF16, D>;
  if (qwaves == S::QW_WIDE)
    return (size_t)make_lay_q<BF16, D, S::QW_WIDE, S::QBC>(mode, has_wk, has_wv, nr, t5_dist, nb,
                                                           want_db)
        .total;
  if (S::BIG && qwaves == S::QW_TINY)
    return (size_t)make_lay_q<BF16, D, S::QW_TINY, S::QBC_TINY>(mode, has_wk, has_wv, nr, t5_dist,
                                                                nb, want_db)
        .total;
  return (size_t)make_lay_q<BF16, D, S::QW_NARROW, S::QBC>(mode, has_wk, has_wv, nr, t5_dist, nb,
                                                           want_db)
      .total;
}
template <bool BF16, int D>
static size_t lds_kv_t(int kqblock, RelMode mode, bool has_wk, bool has_wv, int nr,
                       int t5_dist, int nb) {
  using S = BwdShape<BF16, D>;
  if (kqblock == S::KBQ_WIDE)
    return (size_t)make_lay_kv<BF16, D, S::KW, S::KBQ_WIDE>(mode, has_wk, has_wv, nr, t5_dist, nb)
        .total;
  return (size_t)make_lay_kv<BF16, D, S::KW, S::KBQ_NARROW>(mode, has_wk, has_wv, nr, t5_dist, nb)
      .total;
}

template <bool BF16, int D>
static BwdCfg cfg_t(bool narrow_q, bool narrow_kv, bool tiny_q) {
  using S = BwdShape<BF16, D>;
  if (S::BIG && tiny_q)
    return BwdCfg{S::QW_TINY, S::QBC_TINY, S::KW, narrow_kv ? S::KBQ_NARROW : S::KBQ_WIDE};
  return BwdCfg{narrow_q ? S::QW_NARROW : S::QW_WIDE, S::QBC, S::KW,
                narrow_kv ? S::KBQ_NARROW : S::KBQ_WIDE};
}

BwdCfg bwd_cfg(bool bf16, int d, bool narrow_q, bool narrow_kv, bool tiny_q) {
  if (bf16) {
    if (d > 64) return cfg_t<true, 128>(narrow_q, narrow_kv, false);
    return cfg_t<true, 64>(narrow_q, narrow_kv, tiny_q);
  }
  return cfg_t<false, 64>(narrow_q, narrow_kv, false);
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
static size_t lds_kv_d(int d, int bq, RelMode mode, bool wk, bool wv, int nr, int dist, int nb) {
  switch (d) {
    case 16: return lds_kv_t<BF16, 16>(bq, mode, wk, wv, nr, dist, nb);
    case 32: return lds_kv_t<BF16, 32>(bq, mode, wk, wv, nr, dist, nb);
    case 64: return lds_kv_t<BF16, 64>(bq, mode, wk, wv, nr, dist, nb);
    default: return lds_kv_t<BF16, 128>(bq, mode, wk, wv, nr, dist, nb);
  }
}

size_t bwd_lds_q(bool bf16, int d, const BwdCfg& cfg, RelMode mode, bool has_wk, bool has_wv,
                 int nr, int t5_dist, int nb, bool want_db) {
  return bf16 ? lds_q_d<true>(d, cfg.qwaves, mode, has_wk, has_wv, nr, t5_dist, nb, want_db)
              : lds_q_d<false>(d, cfg.qwaves, mode, has_wk, has_wv, nr, t5_dist, nb, want_db);
}
size_t bwd_lds_kv(bool bf16, int d, const BwdCfg& cfg, RelMode mode, bool has_wk, bool has_wv,
                  int nr, int t5_dist, int nb) {
  return bf16 ? lds_kv_d<true>(d, cfg.kqblock, mode, has_wk, has_wv, nr, t5_dist, nb)
              : lds_kv_d<false>(d, cfg.kqblock, mode, has_wk, has_wv, nr, t5_dist, nb);
}

template <int D, int NW, int BC, bool BF16, int MODE, bool WK, bool WV>
static int launch_q(const BwdParams& p, hipStream_t s) {
  const bool want_db = (MODE == kRelT5 || MODE == kRelGrid || MODE == kRelLabel) &&
                       p.ws_pb != nullptr;
  const LayQ lay = make_lay_q<BF16, D, NW, BC>(MODE, WK, WV, p.nr, p.t5_dist, p.t5.nb, want_db);
  auto kern = bwd_q_kernel<D, NW, BC, BF16, MODE, WK, WV>;
  static std::atomic<int> lds_set[64];
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), lay.total, lds_set);
  if (e != hipSuccess) return (int)e;
  const dim3 grid((unsigned)((int64_t)p.B * p.H * p.n_qtiles));
  hipLaunchKernelGGL(kern, grid, dim3(64 * NW), (size_t)lay.total, s, p);
  return (int)hipGetLastError();
}

template <int D, int NW, int BQ, bool BF16, int MODE, bool WK, bool WV>
static int launch_kv(const BwdParams& p, hipStream_t s) {
  const LayKV lay = make_lay_kv<BF16, D, NW, BQ>(MODE, WK, WV, p.nr, p.t5_dist, p.t5.nb);
  auto kern = bwd_kv_kernel<D, NW, BQ, BF16, MODE, WK, WV>;
  static std::atomic<int> lds_set[64];
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), lay.total, lds_set);
  if (e != hipSuccess) return (int)e;
  const dim3 grid((unsigned)((int64_t)p.B * p.H * p.n_ktiles));
  hipLaunchKernelGGL(kern, grid, dim3(64 * NW), (size_t)max(lay.total, 64 * NW * 4), s, p);
  return (int)hipGetLastError();
}

template <bool BF16, int D, int MODE, bool WK, bool WV>
static int launch_bwd_t(const BwdCfg& cfg, const BwdParams& p, void* stream) {
  using S = BwdShape<BF16, D>;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int e;
  if constexpr (S::BIG && (MODE == kRelShaw || MODE == kRelXL || MODE == kRelGraph) && WK &&
                !WV) {
    if (cfg.qwaves == S::QW_TINY && cfg.qkblock == S::QBC_TINY) {
      e = launch_q<D, S::QW_TINY, S::QBC_TINY, BF16, MODE, WK, WV>(p, s);
      if (e != (int)hipSuccess) return e;
      return cfg.kqblock == S::KBQ_WIDE ? launch_kv<D, S::KW, S::KBQ_WIDE, BF16, MODE, WK, WV>(p, s)
                                        : launch_kv<D, S::KW, S::KBQ_NARROW, BF16, MODE, WK, WV>(p, s);
    }
  }
  if (cfg.qwaves != S::QW_WIDE && cfg.qwaves != S::QW_NARROW) return (int)hipErrorInvalidValue;
  e = cfg.qwaves == S::QW_WIDE ? launch_q<D, S::QW_WIDE, S::QBC, BF16, MODE, WK, WV>(p, s)
                               : launch_q<D, S::QW_NARROW, S::QBC, BF16, MODE, WK, WV>(p, s);
  if (e != (int)hipSuccess) return e;
  e = cfg.kqblock == S::KBQ_WIDE ? launch_kv<D, S::KW, S::KBQ_WIDE, BF16, MODE, WK, WV>(p, s)
                                 : launch_kv<D, S::KW, S::KBQ_NARROW, BF16, MODE, WK, WV>(p, s);
  if (e != (int)hipSuccess) return e;
  return e;
}

template <bool BF16, int D>
static int launch_bwd_mode(const BwdCfg& c, RelMode mode, bool wk, bool wv, const BwdParams& p,
                           void* stream) {
  if (mode == kRelT5) return launch_bwd_t<BF16, D, kRelT5, false, false>(c, p, stream);
  if (mode == kRelGrid) return launch_bwd_t<BF16, D, kRelGrid, false, false>(c, p, stream);
  if (mode == kRelLabel) return launch_bwd_t<BF16, D, kRelLabel, false, false>(c, p, stream);
  if (mode == kRelXL) return launch_bwd_t<BF16, D, kRelXL, true, false>(c, p, stream);
  if (mode == kRelGraph) {
    if (wk && wv) return launch_bwd_t<BF16, D, kRelGraph, true, true>(c, p, stream);
    if (wk) return launch_bwd_t<BF16, D, kRelGraph, true, false>(c, p, stream);
    return launch_bwd_t<BF16, D, kRelGraph, false, true>(c, p, stream);
  }
  if (mode == kRelShaw) {
    if (wk && wv) return launch_bwd_t<BF16, D, kRelShaw, true, true>(c, p, stream);
    if (wk) return launch_bwd_t<BF16, D, kRelShaw, true, false>(c, p, stream);
    return launch_bwd_t<BF16, D, kRelShaw, false, true>(c, p, stream);
  }
  if (mode == kRelNone) return launch_bwd_t<BF16, D, kRelNone, false, false>(c, p, stream);
  return (int)hipErrorInvalidValue;
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
