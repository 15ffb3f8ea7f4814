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
//   O^T += V^T P^T, P^T taken straight from the S^T accumulators; bf16 V^T
//                 fragments come from the row-major V tile by LDS transpose
//                 reads (ds_read_b64_tr_b16).
// Because a lane owns a query, the online-softmax rescale of O, of the row
// sum and of the tail sum is a per-lane multiply; only the row max needs one
// cross-lane exchange per key tile.
//
// Memory pipeline: K and V tiles stream from HBM straight into LDS with
// global_load_lds_dwordx4 (no register staging) through a ring of nstage
// stages, nstage - 1 tiles ahead of the one being used; one workgroup barrier
// per tile.  Tiles are stored row-major with their 16-byte chunks XOR-swizzled
// per row so that MFMA fragment reads and transpose reads are free of LDS
// bank conflicts.  The relative tables (w^K, w^V rows of the reachable
// labels; the T5 bias column of the head) come in the same way.
//
// Relative key term: L is computed once per workgroup by one small MFMA
// product (BR x labels) and kept in LDS, one private row per query.  Inside
// the band |j - i| < c each logit gathers L[i, j-i+c]; outside the band the
// label is -c or +c for the whole tile, so two per-lane registers serve it.
//
// Relative value term: inside the band each label holds exactly one key, so
// its weight is exp(e_ij - m_i): in-band logits are written to a second LDS
// row per query and turned into weights in the epilogue once m_i is final.
// The +c tail is a running sum (empty under the causal mask) and the -c tail
// is what the row sum leaves.  The epilogue adds S W^V with MFMA.
//
// Transformer-XL, fused (XL mode, d <= 64): the relative logit (q_i + v).R_{i-j}
// is formed per key tile instead of once per query row: each wave multiplies
// its 32 queries by the BC + 31 position-table rows of the distances they can
// reach in the tile (rows read straight from L2 as MFMA operands), stores the
// products position-major in a per-wave LDS block and gathers them like the
// band.  No per-query window of every distance is kept, so long windows leave
// room for four-wave workgroups.
//
// Edge labels (label mode): the scalar bias is indexed by a label given per
// (query, key) pair instead of a function of the offset.  Each wave's 32 rows
// of a tile's label matrix travel with the K/V stage by LDS-DMA, and every
// logit gathers its bias from the head's row of the table in LDS.
//
// Edge labels with key and value tables (graph mode): Eq. 4 and Eq. 3 with
// a^K_ij = w^K[label], a^V_ij = w^V[label].  The relative logits are the Shaw
// rows over the NL labels; the label tiles travel as in label mode.  A label
// may hold any number of a row's keys, so the value term keeps a second LDS row
// per query and wave half, S[i, r] = sum of p_ij over the half's keys of label r
// (each half owns its row, so plain LDS read-modify-writes suffice: LDS float
// atomics measured about three times slower per call here), rescaled with the
// row when the running max grows; the epilogue adds (S_0 + S_1) W^V.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "relattn_device.h"
#include "relattn_internal.h"
#include "relattn_tiles.h"

namespace relattn {

// A row max may run ahead of the max used for the exponentials by this much
// (log2 units) before the running sums are rescaled: p <= 2^8 stays exact in
// fp32 sums and in bf16 operands, and most tiles then skip the rescale.
constexpr float kRescaleSlack = 8.f;

// ---------------------------------------------------------------------------
// Geometry and LDS budget, identical on host and device.
// ---------------------------------------------------------------------------

template <bool BF16, int D, int NW, int BC>
struct Geo {
  using T = std::conditional_t<BF16, __bf16, float>;
  static constexpr int ESZ = sizeof(T);
  static constexpr int BR = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int NKB = BC / 32;             // 32-key blocks per tile
  static constexpr int DVB = (D + 31) / 32;       // 32-wide d_v blocks
  static constexpr int KSTEP = BF16 ? 16 : 2;     // contraction per MFMA
  static constexpr int NKS = D / KSTEP;           // MFMAs over d
  static constexpr int ROWB = D * ESZ;            // bytes per K/V row
  static constexpr int TILEB = BC * ROWB;         // one K or V tile
  static constexpr int STAGEB = 2 * TILEB;        // K then V
  static constexpr int LPW = STAGEB / 1024 / NW;  // DMA instructions per wave per stage
  // A lane's logits come in groups of 8 keys KSTR apart, spanning SPAN
  // offsets.  Relative-logit rows hold the reachable labels with PADL copies
  // of the first label below and PADU copies of the last above: a group then
  // reads its 8 entries from one base clamped to [0, labels + PADL + PADU -
  // SPAN], whether it lies in the band, in a tail or across an edge, and the
  // top SPAN entries stay clear of the band-logit stores (which reach at most
  // SPAN - 1 entries past the last label).
  static constexpr int KSTR = BF16 ? 1 : 2;
  static constexpr int SPAN = 7 * KSTR + 1;
  static constexpr int PADL = SPAN - 1;
  static constexpr int PADU = 2 * SPAN - 1;
  // fused XL: 32-distance MFMA blocks per key tile (the BC + 31 offsets a
  // wave's 32 queries reach in a tile), and the per-wave LDS block of their
  // products (position-major, XRS floats per position)
  static constexpr int NXB = (BC + 62) / 32;
  static constexpr int XRS = 34;
  static constexpr int XLB = NXB * 32 * XRS * 4;
  static_assert(STAGEB % (1024 * NW) == 0, "stage must split into whole 1 KB instructions");
  static_assert(BR * ROWB % 1024 == 0, "the Q tile must split into whole 1 KB instructions");
};

struct Layout {
  int wk, wv, le, tbc, tb, qs, lab, total;  // byte offsets / total bytes
  int wk_rows, wv_rows, lrs;       // tile rows, relative-row stride (floats)
  int wk_chunk;                    // w^K rows staged at a time (multiple of 32)
  int wv_chunk;                    // w^V rows staged at a time (multiple of 16)
  int se, ses;                     // graph mode: weight-sum rows, their stride (floats)
};

// w^V staging (wv_mode): kWvResident gives the tile its own region, loaded
// in the prologue; kWvRing loads it into the first ring stage the loop no
// longer needs (it must fit one stage); kWvChunked stages it in chunks
// through the free ring after the loop.
template <bool BF16, int D, int NW, int BC>
__host__ __device__ inline Layout make_layout(int mode, bool has_wk, bool has_wv, int nr,
                                              int nstage, int t5_dist, int t5_nb, int wv_mode) {
  using G = Geo<BF16, D, NW, BC>;
  Layout L{};
  int off = nstage * G::STAGEB;
  auto take = [&](int bytes) {
    const int at = off;
    off += (bytes + 15) & ~15;
    return at;
  };
  const bool graph = mode == kRelGraph;
  const bool shaw = mode == kRelShaw || graph, t5 = mode == kRelT5 || mode == kRelGrid;
  const bool lab = mode == kRelLabel, xlf = mode == kRelXL;
  L.wk_rows = dma_rows((nr + 31) & ~31, G::ROWB);
  L.wv_rows = dma_rows((nr + 15) & ~15, G::ROWB);
  // relative row: padding, nr labels, padding.  Dword LDS accesses are
  // served 32 lanes at a time by 32 banks; the lanes of a wave hold 32
  // consecutive queries and read their rows along a diagonal j - i (or, once
  // clamped, down a column).  A stride of 2 mod 4 keeps both patterns, and
  // the two dwords of each ds_read2/ds_write2, nearly free of bank conflicts
  // (measured: a stride of 0 mod 8 costs about five times as many).
  {
    const int m = nr + G::PADL + G::PADU;
    L.lrs = m + ((2 - m) & 3);
  }
  // the w^K tile is read once, before the loop, in label blocks of 32: it is
  // staged in the last ring stage, which receives its first K/V tile only
  // inside the loop (in several chunks if it does not fit)
  L.wk = (nstage - 1) * G::STAGEB;
  L.wk_chunk = min(L.wk_rows, (G::STAGEB / G::ROWB) / 32 * 32);
  L.wv = 0;
  L.wv_chunk = L.wv_rows;
  if (shaw && has_wv && wv_mode == kWvResident) {
    L.wv = take(L.wv_rows * G::ROWB);
  } else if (shaw && has_wv && wv_mode == kWvChunked) {
    L.wv_chunk = min(L.wv_rows, (nstage * G::STAGEB / G::ROWB) / 16 * 16);
  }
  // The Q tile of the workgroup arrives by LDS-DMA and is read into registers
  // in the prologue: it borrows the relative rows (written only afterwards),
  // or else the last ring stage, which the loop fills first, or else (too
  // big for a stage) a region of its own.
  const int q_bytes = G::BR * G::ROWB;
  if (shaw && (has_wk || has_wv)) {
    L.le = take(max(G::BR * L.lrs * 4, q_bytes));
    L.qs = L.le;
  } else {
    L.le = off;
    L.qs = q_bytes <= G::STAGEB ? (nstage - 1) * G::STAGEB : take(q_bytes);
    // fused XL: per wave, the tile's relative logits position-major, 32 lanes
    // (+2 floats) per position
    if (xlf) L.le = take(NW * G::XLB);
  }
  L.tbc = (t5 || lab) ? take(((t5_nb + 63) & ~63) * 4) : off;
  L.tb = t5 ? take((2 * t5_dist + 1 + G::PADL + G::PADU) * 4) : off;
  // label and graph modes: one BR x BC byte tile of labels per ring stage
  L.lab = (lab || graph) ? take(nstage * G::BR * BC) : off;
  // graph mode: per query and wave half, the weight sum of each label (odd
  // stride: the lanes' rows start in different banks)
  L.ses = nr | 1;
  L.se = (graph && has_wv) ? take(2 * G::BR * L.ses * 4) : off;
  L.total = off;
  return L;
}

// Waves per SIMD the register budget is sized for (the host plan uses the
// same rule): d = 128 with 64-key tiles needs the whole register file for one,
// with 32-key tiles (bf16) two fit; for d <= 64, three for bf16 without the
// Shaw tables (168 registers; lets the T5 grid run in one round) when that
// compiles without spilling (d <= 32, or four-wave workgroups, whose
// per-wave share of the stage loads is smallest), and two otherwise.
template <int D, int NW, int MODE, bool BF16, int BC>
__host__ __device__ constexpr int waves_per_simd() {
  return D > 64 ? ((BF16 && BC == 32) ? 2 : 1)
                : ((BF16 && MODE != kRelShaw && MODE != kRelXL && MODE != kRelGraph &&
                    (D <= 32 || NW == 4)) ? 3 : 2);
}
template <int D, int NW, int BC, bool BF16, int MODE, bool HAS_WK, bool HAS_WV>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(waves_per_simd<D, NW, MODE, BF16, BC>()))) void fwd_kernel(
    const FwdParams p) {
  using G = Geo<BF16, D, NW, BC>;
  using T = typename G::T;
  using Op = std::conditional_t<BF16, bf16x8, float>;
  constexpr int NT = G::NT, NKB = G::NKB, DVB = G::DVB;
  constexpr int NKS = G::NKS, ROWB = G::ROWB, LPW = G::LPW;
  constexpr int KSTR = G::KSTR, SPAN = G::SPAN, PADL = G::PADL, PADU = G::PADU;
  constexpr bool GRAPH = (MODE == kRelGraph);  // Shaw tables indexed by per-pair labels
  constexpr bool SHAW = (MODE == kRelShaw) || GRAPH;
  constexpr bool GRID = (MODE == kRelGrid);  // the bias by 2-D offset
  constexpr bool T5 = (MODE == kRelT5) || GRID;
  constexpr bool LAB = (MODE == kRelLabel);
  constexpr bool XLF = (MODE == kRelXL);  // fused Transformer-XL
  constexpr bool GATHER = (SHAW && HAS_WK) || T5 || LAB || XLF;  // a gathered relative logit
  constexpr int NXB = G::NXB, XRS = G::XRS;
  // label mode: each wave loads its 32 rows of a tile's labels (32 x BC bytes)
  // with the stage, in 1 KB instructions
  constexpr int LLPW = (LAB || GRAPH) ? BC / 32 : 0;
  constexpr int SLPW = LPW + LLPW;  // DMA instructions per wave per stage
  constexpr int LABB = G::BR * BC;  // label bytes per stage

  // One field of each 64-byte line of the parameter block (and the grid size),
  // so that all of them are requested together behind one wait instead of
  // one scalar-cache miss after another as the prologue first needs them.
  asm volatile("" ::"s"(p.q), "s"(p.q_sb), "s"(p.v_sn), "s"(p.tb_sb), "s"(p.dma32), "s"(gridDim.x));
  // ---- which tile
  int bh, qt;
  constexpr int kCusPerXcd = 32;
  if (p.causal && (gridDim.x & 7) == 0 && p.n_qtiles == kCusPerXcd &&
      (gridDim.x >> 3) % (2 * kCusPerXcd) == 0) {
    // A head has one causal tile per CU of its XCD: the XCD takes its heads two
    // at a time and deals the pair's tiles heaviest first, alternating between
    // the two heads, so only two heads' K and V are in use at a time (they fit
    // the XCD's L2 where every head of the XCD at once did not).
    const int x = blockIdx.x & 7, loc = blockIdx.x >> 3;
    const int pair = loc / (2 * kCusPerXcd), k = loc % (2 * kCusPerXcd);
    const int hpx = (gridDim.x >> 3) / p.n_qtiles;  // heads per XCD
    bh = x * hpx + 2 * pair + (k & 1);
    qt = p.n_qtiles - 1 - (k >> 1);
  } else if (p.causal && (gridDim.x & 7) == 0 && (gridDim.x >> 3) % p.n_qtiles == 0) {
    // Causal tiles differ in work.  Each XCD holds whole heads; it is dealt the
    // heaviest tile of each of its heads first, then the next heaviest, and so
    // on, so that the workgroups that share a CU in one round differ in work
    // and later rounds start with the longest remaining tiles.
    const int x = blockIdx.x & 7, loc = blockIdx.x >> 3;
    const int hpx = (gridDim.x >> 3) / p.n_qtiles;  // heads per XCD
    const int rank = loc / hpx;
    bh = x * hpx + (loc - rank * hpx);
    qt = p.n_qtiles - 1 - rank;
  } else {
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    bh = lid / p.n_qtiles;
    qt = lid - bh * p.n_qtiles;
    if (p.causal) qt = p.n_qtiles - 1 - qt;  // longest causal rows first
  }
  // (b, h) of the tile: batch entry major; in the XL mode head major instead,
  // so that the heads' position tables, shared by every batch entry, are read
  // by one XCD each (an XCD holds consecutive ids) rather than by all of them
  int b, h;
  if constexpr (XLF) {
    h = bh / p.B;
    b = bh - h * p.B;
  } else {
    b = bh / p.H;
    h = bh - b * p.H;
  }
  const int i0 = qt * (32 * NW);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loops
  const int ql = lane & 31, hh = lane >> 5;
  const int qrow = wave * 32 + ql;
  const int qi = i0 + qrow;
  const bool q_ok = qi < p.n;
  const int wq0 = i0 + wave * 32;
  const int c = p.clip;
  const int r_hi = p.r_lo + p.nr - 1;
  const int nstage = p.nstage;
  const bool wv_ring = SHAW && HAS_WV && p.wv_mode == kWvRing;

  const Layout lay = make_layout<BF16, D, NW, BC>(MODE, HAS_WK, HAS_WV, p.nr, nstage, p.t5_dist,
                                                  p.t5.nb, p.wv_mode);
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char RELATTN_LDS* smem_lds = (unsigned char RELATTN_LDS*)smem;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem_lds;  // LDS byte address of smem
  float* LE = reinterpret_cast<float*>(smem + lay.le);
  float* TBC = reinterpret_cast<float*>(smem + lay.tbc);
  float* TB = reinterpret_cast<float*>(smem + lay.tb);
  float* myLE = LE + qrow * lay.lrs;

  const T* qg = reinterpret_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const T* kg = reinterpret_cast<const T*>(p.k) + b * p.k_sb + h * p.k_sh;
  const T* vg = reinterpret_cast<const T*>(p.v) + b * p.v_sb + h * p.v_sh;
  T* og = reinterpret_cast<T*>(p.o) + b * p.o_sb + h * p.o_sh;
  const uint8_t* labg = (LAB || GRAPH) ? p.lab + b * p.lab_sb : nullptr;

  // ---- LDS-DMA, oldest first: the Q tile, the relative tables, then the
  // first K/V stages.  (Q goes through LDS too: the compiler cannot count the
  // DMA instructions issued after a register load and would wait for all of
  // them before the first use of Q.)  Query rows past n and key rows past the
  // key length read the last valid row (finite, never stored or masked).
  // Transformer-XL: this lane's half of the head's global biases u (content
  // logit) and v (relative logit), requested before any LDS-DMA so that the
  // counted DMA waits below stay exact.
  Op xu[NKS], xv[NKS];
  if constexpr ((SHAW && HAS_WK) || XLF) {
    if (XLF || p.xl) {
      const T* up = reinterpret_cast<const T*>(p.xl_u) + h * p.xl_u_sh;
      const T* vp = reinterpret_cast<const T*>(p.xl_v) + h * p.xl_v_sh;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if constexpr (BF16) {
          xu[ks] = *reinterpret_cast<const bf16x8*>(up + 16 * ks + 8 * hh);
          xv[ks] = *reinterpret_cast<const bf16x8*>(vp + 16 * ks + 8 * hh);
        } else {
          xu[ks] = up[2 * ks + hh];
          xv[ks] = vp[2 * ks + hh];
        }
      }
    }
  }
  compiler_fence();
  dma_tile<ROWB, NW>(smem_lds + lay.qs, qg, p.q_sn, i0, p.n - 1, G::BR, wave, lane);
  compiler_fence();
  const T* wkh = reinterpret_cast<const T*>(p.wk) + h * p.wk_sh;
  const T* wvh = reinterpret_cast<const T*>(p.wv) + h * p.wv_sh;
  int n_after_q = 0;  // this wave's DMA instructions issued after the Q tile
  if constexpr (SHAW && HAS_WK) {
    n_after_q += dma_tile<ROWB, NW>(smem_lds + lay.wk, wkh, p.wk_sr, p.r_lo, r_hi, lay.wk_chunk,
                                    wave, lane);
  }
  compiler_fence();
  int n_after_wk = 0;  // this wave's DMA instructions issued after the w^K chunk
  if constexpr (SHAW && HAS_WV) {
    if (p.wv_mode == kWvResident)
      n_after_wk += dma_tile<ROWB, NW>(smem_lds + lay.wv, wvh, p.wv_sr, p.r_lo, r_hi,
                                       lay.wv_rows, wave, lane);
  }
  if constexpr (T5 || LAB) {
    // bias column of this head (or the window of its row of a table by
    // offset, or its row of a table by label), 4 bytes per lane, issued by
    // wave 0
    if (wave == 0) {
      for (int I = 0; I * 64 < p.t5.nb; ++I) {
        const int bucket = min(I * 64 + lane, p.t5.nb - 1) + p.ob_lo;
        __builtin_amdgcn_global_load_lds(
            (const RELATTN_GLOBAL void*)(p.t5_bias + bucket * p.tb_sb + h * p.tb_sh),
            (RELATTN_LDS void*)(smem_lds + lay.tbc + I * 256), 4, 0, 0);
      }
    }
  }
  compiler_fence();
  // Key range of this workgroup.  The key length is read only now, after the
  // Q and table requests have left, as a scalar load through the constant
  // address space: a vector load would be counted with the DMA loads, and any
  // earlier scalar load would be waited for together with the kernel arguments
  // that the first requests need.  The opaque move keeps the compiler from
  // hoisting the load.
  int kv_len = p.n;
  if (p.key_lens) {
    const int32_t* klp = p.key_lens + b;
    asm volatile("" : "+s"(klp));
    kv_len = min(max(*(const RELATTN_CONST int32_t*)klp, 0), p.n);
  }
  const int kv_end = p.causal ? min(kv_len, i0 + 32 * NW) : kv_len;
  const int kv_last = max(kv_len - 1, 0);
  const int ntiles = (kv_end + BC - 1) / BC;
  uint32_t soff[LPW];  // per-lane offsets of this wave's stage loads (fast path)
  if (p.dma32) stage_offsets<ROWB, NW, BC, T>(soff, p.k_sn, p.v_sn, wave, lane);
  auto issue_stage = [&](int tile, int stage) __attribute__((always_inline)) {
    if (p.dma32 && tile * BC + BC - 1 <= kv_last) {
      dma_stage_fast<ROWB, NW, BC>(smem_lds + stage * G::STAGEB, kg + (int64_t)tile * BC * p.k_sn,
                                   vg + (int64_t)tile * BC * p.v_sn, soff, wave);
    } else {
      dma_stage<ROWB, NW, BC>(smem_lds + stage * G::STAGEB, kg, p.k_sn, vg, p.v_sn, tile * BC,
                              kv_last, wave, lane);
    }
    if constexpr (LAB || GRAPH) {
      // this wave's rows of the tile's labels, stored chunk-major: the 16-byte
      // chunk c (keys 16c ..) of row r at slot 32 c + r, so that the 32 rows
      // of one chunk are 512 contiguous bytes.  Rows past n read row n - 1;
      // chunks past the last one holding a key read that chunk.
      unsigned char RELATTN_LDS* dst = smem_lds + lay.lab + stage * LABB + wave * (32 * BC);
      const int col_max = ((p.n - 1) >> 4) << 4;
#pragma unroll
      for (int I = 0; I < LLPW; ++I) {
        const int slot = I * 64 + lane;
        const int row = min(wq0 + (slot & 31), p.n - 1);
        const int col = min(tile * BC + 16 * (slot >> 5), col_max);
        __builtin_amdgcn_global_load_lds(
            (const RELATTN_GLOBAL void*)(labg + (int64_t)row * p.lab_sn + col),
            (RELATTN_LDS void*)(dst + I * 1024), 16, 0, 0);
      }
    }
    compiler_fence();
  };
  const int n_pre = min(nstage - 1, ntiles);
  for (int s = 0; s < n_pre; ++s) issue_stage(s, s);
  n_after_wk += n_pre * SLPW;
  n_after_q += n_after_wk;

  // ---- Q as the B operand of S^T = K Q^T, in registers for the whole kernel
  wait_vm_dyn(SHAW && HAS_WK ? n_after_wk : ((T5 || LAB) ? n_pre * SLPW : n_after_q));
  block_sync();  // every wave's share of the Q tile (and of the tables) landed
  Op qop[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if constexpr (BF16) {
      qop[ks] = frag_row<ROWB>(smem + lay.qs, qrow, 2 * ks + hh);
    } else {
      qop[ks] = elem_f32<ROWB>(smem + lay.qs, qrow, 2 * ks + hh);
    }
  }
  if constexpr (SHAW && (HAS_WK || HAS_WV)) block_sync();  // Q sits in the relative rows
  // fused XL: q + v for the relative logit, q + u for the content logit
  Op qpos_x[NKS];
  if constexpr (XLF) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qpos_x[ks] = op_add(qop[ks], xv[ks]);
      qop[ks] = op_add(qop[ks], xu[ks]);
    }
  }
  const T* xrh = XLF ? reinterpret_cast<const T*>(p.wk) + h * p.wk_sh : nullptr;

  // ---- relative logits in LDS.  Shaw: row qrow holds scale*log2e*q.w^K_r for
  // the reachable label rows r_lo..r_hi at entries PADL + (r - r_lo), with
  // PADL copies of the first label below and PADU copies of the last above.
  // T5: one shared vector holds log2e*bias[beta(delta), h] for delta in
  // [-dist, dist] at entries PADL + dist + delta, padded the same way.
  if constexpr (SHAW && HAS_WK) {
    // the relative logit takes q + v under Transformer-XL
    Op qpos[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qpos[ks] = p.xl ? op_add(qop[ks], xv[ks]) : qop[ks];
    const unsigned char* wkt = smem + lay.wk;
    const int nlb = (p.nr + 31) / 32;
    float edge_lo = 0.f;
    const int lb_chunk = lay.wk_chunk / 32;
    for (int lb = 0; lb < nlb; ++lb) {
      if (lb > 0 && lb % lb_chunk == 0) {
        // next chunk of w^K rows (only when the table exceeds one ring stage)
        block_sync();
        dma_tile<ROWB, NW>(smem_lds + lay.wk, wkh, p.wk_sr, p.r_lo + lb * 32, r_hi, lay.wk_chunk,
                           wave, lane);
        wait_vm<0>();
        block_sync();
      }
      const int row = (lb % lb_chunk) * 32 + ql;  // MFMA row m = ql <-> label r_lo + lb*32 + ql
      Op a[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if constexpr (BF16) {
          a[ks] = frag_row<ROWB>(wkt, row, 2 * ks + hh);
        } else {
          a[ks] = elem_f32<ROWB>(wkt, row, 2 * ks + hh);
        }
      }
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc = mfma(a[ks], qpos[ks], acc);
      if (PADL + nlb * 32 <= lay.lrs) {
        // the whole 32-label block fits the row: entries past the last label
        // land in the padding, which is written below
#pragma unroll
        for (int i = 0; i < 16; ++i)
          myLE[PADL + lb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3)] = acc[i] * p.scale_log2;
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int idx = lb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (idx < p.nr) myLE[PADL + idx] = acc[i] * p.scale_log2;
        }
      }
      if (lb == 0) edge_lo = acc[0] * p.scale_log2;  // label 0 of this lane's query (hh = 0)
    }
    // the content logit takes q + u under Transformer-XL
    if (p.xl) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qop[ks] = op_add(qop[ks], xu[ks]);
    }
    compiler_fence();  // the row was written by both halves of this wave
    // Under the causal mask no offset above 0 is visible: the upper padding
    // holds -inf, so every logit gathered for a future key comes out masked.
    const float edge = hh ? (p.causal ? kNegInf : myLE[PADL + p.nr - 1]) : edge_lo;
    float* pad = myLE + (hh ? PADL + p.nr : 0);
    const int npad = hh ? PADU : PADL;
#pragma unroll
    for (int x = 0; x < PADU; ++x)
      if (x < npad) pad[x] = edge;
    compiler_fence();
  }
  if constexpr (T5) {
    const int nb = 2 * p.t5_dist + 1 + PADL + PADU;
    for (int x = tid; x < nb; x += NT) {
      const int delta = min(max(x - PADL - p.t5_dist, -p.t5_dist), p.t5_dist);
      // as for the Shaw rows: future offsets carry the causal mask
      const int entry = p.ob ? delta + p.t5_dist : t5_bucket(delta, p.t5);
      TB[x] = (p.causal && x - PADL - p.t5_dist > 0) ? kNegInf : kLog2e * TBC[entry];
    }
    block_sync();
  }
  if constexpr (LAB) {
    // the head's bias row in log2 units, gathered by label in the loop
    for (int x = tid; x < p.t5.nb; x += NT) TBC[x] *= kLog2e;
    block_sync();
  }

  // graph mode: this lane's weight-sum row (row 2 qrow + hh) starts at zero
  float* myS = reinterpret_cast<float*>(smem + lay.se) + (2 * qrow + hh) * lay.ses;
  if constexpr (GRAPH && HAS_WV) {
    for (int r = 0; r < p.nr; ++r) myS[r] = 0.f;
  }

  // window of offsets delta = j - i covered by the relative row, and the
  // relative logit of its two ends (used for tiles entirely outside the band)
  const int dlo = T5 ? -p.t5_dist : p.r_lo - c;  // delta of entry PADL
  const int nwin = T5 ? 2 * p.t5_dist + 1 : p.nr;
  const int gtop = nwin + PADL + PADU - SPAN;     // highest gather base
  const float* relrow = T5 ? TB : myLE;
  float Llo = 0.f, Lhi = 0.f;
  if constexpr (GATHER && !LAB && !XLF) {
    Llo = relrow[PADL];
    Lhi = relrow[PADL + nwin - 1];
  }
  const int band = T5 ? p.t5_dist : c;  // |j - i| >= band: one end value for the tile
  // 2-D window bias: this lane's query on the M x M grid
  int gy = 0, gx = 0;
  if constexpr (GRID) {
    const int qc = min(qi, p.n - 1);
    gy = qc / p.grid_m;
    gx = qc - gy * p.grid_m;
  }
  // offsets whose label holds a single key (1 <= r <= 2c - 1, reachable):
  // their logits are kept for the value term
  const int wb_lo = max(1, p.r_lo) - c, wb_hi = min(2 * c - 1, r_hi) - c;

  // ---- running state (per lane: one query, half of each tile's keys)
  f32x16 oacc[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) oacc[mb] = f32x16{};
  float m_run = kNegInf;
  float l_part = 0.f, thi = 0.f;
  // transpose-read lane bases of the V tile (columns 32 mb ..)
  uint32_t trb_lo[DVB], trb_hi[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) frag_col_base<ROWB, D>(32 * mb, lane, trb_lo[mb], trb_hi[mb]);
  const int hi_from = max(c, 1 - c);    // offsets >= hi_from fall in the +c bucket
  const int hoff = BF16 ? 8 * hh : hh;  // key offset of this lane half
  int wv_stage = -1, wv_cnt = 0;        // ring stage and DMA count of the w^V tile

  // Start of tile t: the tile landed for this wave (later stages and w^V may
  // still be in flight), then for every wave, which frees stage (t - 1) %
  // nstage for the next request.  `act`: the wave computes the tile.
  using XrOps = Op[XLF ? NXB : 1][NKS];
  auto tile_head = [&](int t, int st_next, bool act, XrOps& xr) __attribute__((always_inline)) {
    const int j0 = t * BC;
    {
      // the steady state (one stage still in flight) and the drained state
      // take one compare each instead of the general switch's branch tree
      const int pending = min(nstage - 2, ntiles - 1 - t) * SLPW + wv_cnt;
      if (pending == SLPW) wait_vm<SLPW>();
      else if (pending == 0) wait_vm<0>();
      else wait_vm_dyn(pending);
    }
    block_sync();
    // fused XL: the position-table rows of the distances this wave reaches in
    // the tile, as MFMA A operands (row = MFMA row ql of block b: offset j - i
    // = omin + 32 b + ql, distance i - j clamped to the window), requested
    // before the next stage so that one counted wait covers them
    if constexpr (XLF) {
      if (act) {
        const int omin = j0 - wq0 - 31;
#pragma unroll
        for (int bx = 0; bx < NXB; ++bx) {
          const int dist = min(max(-(omin + 32 * bx + ql), -c), c);
          const T* rp = xrh + (int64_t)dist * p.wk_sr;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            if constexpr (BF16) {
              xr[bx][ks] = *reinterpret_cast<const bf16x8*>(rp + 16 * ks + 8 * hh);
            } else {
              xr[bx][ks] = rp[2 * ks + hh];
            }
          }
        }
      }
    }
    if (t + nstage - 1 < ntiles) {
      issue_stage(t + nstage - 1, st_next);
    } else if (wv_ring && wv_stage < 0) {
      // no K/V tile left to prefetch: the free stage takes the w^V rows
      wv_stage = st_next;
      wv_cnt = dma_tile<ROWB, NW>(smem_lds + wv_stage * G::STAGEB, wvh, p.wv_sr, p.r_lo, r_hi,
                                  lay.wv_rows, wave, lane);
      compiler_fence();
    }
  };
  // The tiles this wave computes are a prefix: none when it holds no live
  // query, under the causal mask those up to its last row.  The rest only
  // keep the workgroup's waits, barriers and requests in step.  (Two loops
  // rather than a skip inside one: a path around the tile's work made the
  // compiler copy every accumulator at the loop's back edge.)
  const int t_act = (wq0 >= p.n) ? 0 : (p.causal ? min(ntiles, (wq0 + 31) / BC + 1) : ntiles);
  int st_cur = 0, st_next = nstage - 1;  // ring stages of tiles t and t + nstage - 1
  int t = 0;
  for (; t < t_act; ++t, st_cur = (st_cur + 1 == nstage) ? 0 : st_cur + 1,
                    st_next = (st_next + 1 == nstage) ? 0 : st_next + 1) {
    const int j0 = t * BC;
    XrOps xr;
    tile_head(t, st_next, true, xr);

    const unsigned char* Kt = smem + st_cur * G::STAGEB;
    const unsigned char* Vt = Kt + G::TILEB;

    // S^T block kb: rows = keys j0 + 32kb + .., columns = this wave's queries
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int krow = 32 * kb + k_row_of_mfma_row<BF16>(ql);
      Op a[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if constexpr (BF16) {
          a[ks] = frag_row<ROWB>(Kt, krow, 2 * ks + hh);
        } else {
          a[ks] = elem_f32<ROWB>(Kt, krow, 2 * ks + hh);
        }
      }
      s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) s[kb] = mfma(a[ks], qop[ks], s[kb]);
    }

    // fused XL: relative logits of the tile's distances, position p = offset
    // - omin at xw[p * XRS + lane's query]
    if constexpr (XLF) {
      // the table rows are older than this iteration's stage requests
      if (t + nstage - 1 < ntiles) wait_vm<SLPW>();
      else wait_vm<0>();
      float* xw = reinterpret_cast<float*>(smem + lay.le) + wave * (NXB * 32 * XRS) + ql;
#pragma unroll
      for (int bx = 0; bx < NXB; ++bx) {
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) acc = mfma(xr[bx][ks], qpos_x[ks], acc);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          xw[(32 * bx + 8 * (i >> 2) + 4 * hh + (i & 3)) * XRS] = acc[i] * p.scale_log2;
      }
      compiler_fence();  // both halves of the wave wrote each query's column
    }

    // Register (kb, 8g + e) holds key j0 + hoff + 32kb + 16g + KSTR*e, i.e.
    // offset delta = kofs + 32kb + 16g + KSTR*e from this lane's query.
    const int kofs = j0 + hoff - qi;
    const int dmin = j0 - (wq0 + 31), dmax = j0 + BC - 1 - wq0;
    const bool all_lo = dmax <= -band, all_hi = dmin >= band;  // wave-uniform
    const bool off_band = ((SHAW && !GRAPH) || T5) && (all_lo || all_hi);
    // Per-element masking: key-length cuts, and causal cuts unless the
    // gathered relative logits already carry them (-inf past offset 0; not
    // so for labels).
    const bool causal_cut = p.causal && j0 + BC - 1 > wq0;
    const bool need_mask =
        (j0 + BC > kv_len) ||
        (causal_cut && (LAB || XLF || GRAPH || !(GATHER && !off_band)));
    // visible iff its key offset within the lane's keys is <= lim
    const int lim = min(kv_len - 1 - j0 - hoff, p.causal ? -kofs : 0x3fffffff);

    // graph mode: the lane's label chunks of the tile (two 16-key chunks per
    // 32-key block), for the key-table gather and the value-term sums
    uint4 glw[GRAPH ? NKB : 1][2];
    if constexpr (GRAPH) {
      const unsigned char* labt = smem + lay.lab + st_cur * LABB + wave * (32 * BC);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int g = 0; g < 2; ++g)
          glw[kb][g] = *reinterpret_cast<const uint4*>(labt + ((2 * kb + g) * 32 + ql) * 16);
    }
    // label of register (kb, 8g + e), clamped to the table
    auto glabel = [&](int kb, int g, int e) __attribute__((always_inline)) {
      const uint4 w4 = glw[GRAPH ? kb : 0][g];
      uint32_t byte;
      if constexpr (BF16) {
        const uint32_t dw = (e < 4) ? (hh ? w4.z : w4.x) : (hh ? w4.w : w4.y);
        byte = (dw >> (8 * (e & 3))) & 0xffu;
      } else {
        const uint32_t dw = (e < 2) ? w4.x : (e < 4) ? w4.y : (e < 6) ? w4.z : w4.w;
        byte = (dw >> (8 * (hh + 2 * (e & 1)))) & 0xffu;
      }
      return min((int)byte, p.nr - 1);
    };

    // logits (log2 units) of the tile, masked to -inf where invisible
    float tmax = kNegInf;
    auto finish = [&](float (&rv)[NKB][16], auto mask_tag) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ko = 32 * kb + 16 * (i >> 3) + KSTR * (i & 7);
          float x = fmaf(s[kb][i], p.scale_log2, rv[kb][i]);
          if constexpr (MASK) x = (ko <= lim) ? x : kNegInf;
          s[kb][i] = x;
          tmax = fmaxf(tmax, x);
        }
    };
    // one relative logit for every key of the tile (the lane's end value)
    auto finish_const = [&](float rel, auto mask_tag) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ko = 32 * kb + 16 * (i >> 3) + KSTR * (i & 7);
          float x = fmaf(s[kb][i], p.scale_log2, rel);
          if constexpr (MASK) x = (ko <= lim) ? x : kNegInf;
          s[kb][i] = x;
          tmax = fmaxf(tmax, x);
        }
    };
    if (!GATHER || off_band) {
      // no gathered term: nothing relative, or the tile's end value
      const float rel = GATHER ? (all_lo ? Llo : Lhi) : 0.f;
      if (need_mask) {
        finish_const(rel, std::true_type{});
      } else {
        finish_const(rel, std::false_type{});
      }
    } else {
      float rv[NKB][16];
      if constexpr (LAB) {
        // edge labels: the bias of each key's label, from the 16-byte label
        // chunk of the lane's row that holds 16 consecutive keys of the tile
        const unsigned char* labt = smem + lay.lab + st_cur * LABB + wave * (32 * BC);
        const int nbm = p.t5.nb - 1;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const uint4 w4 = *reinterpret_cast<const uint4*>(labt + ((2 * kb + g) * 32 + ql) * 16);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              uint32_t byte;
              if constexpr (BF16) {
                // keys 8 hh + e of the chunk
                const uint32_t dw = (e < 4) ? (hh ? w4.z : w4.x) : (hh ? w4.w : w4.y);
                byte = (dw >> (8 * (e & 3))) & 0xffu;
              } else {
                // keys hh + 2 e of the chunk
                const uint32_t dw = (e < 2) ? w4.x : (e < 4) ? w4.y : (e < 6) ? w4.z : w4.w;
                byte = (dw >> (8 * (hh + 2 * (e & 1)))) & 0xffu;
              }
              rv[kb][8 * g + e] = TBC[min((int)byte, nbm)];
            }
          }
      } else if constexpr (GRAPH) {
        // graph mode: the relative logit of each key's label
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) rv[kb][8 * g + e] = myLE[PADL + glabel(kb, g, e)];
      } else if constexpr (XLF) {
        // fused XL: key group (kb, g) starts at position hoff + 32 kb + 16 g
        // + 31 - ql of the wave's block (offset kofs + 32 kb + 16 g - omin)
        const float* xw =
            reinterpret_cast<const float*>(smem + lay.le) + wave * (NXB * 32 * XRS) + ql;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int p0 = hoff + 32 * kb + 16 * g + 31 - ql;
#pragma unroll
            for (int e = 0; e < 8; ++e) rv[kb][8 * g + e] = xw[(p0 + KSTR * e) * XRS];
          }
      } else if constexpr (GRID) {
        // 2-D window: the bias of the key's offset (dy, dx) from the query,
        // tokens in raster order on an M x M grid; the row of key j is
        // floor((j + 1/2) / M), exact in fp32 for j < 2^22
        const int M = p.grid_m;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = j0 + hoff + 32 * kb + 16 * (i >> 3) + KSTR * (i & 7);
            const int yj = (int)(((float)j + 0.5f) * p.grid_inv);
            const int xj = j - yj * M;
            const int e = (yj - gy + M - 1) * (2 * M - 1) + (xj - gx + M - 1);
            rv[kb][i] = kLog2e * TBC[min(max(e, 0), p.t5.nb - 1)];
          }
      } else {
        // band: every relative logit of the tile, 8 entries per group read
        // from one clamped base (the row padding makes the clamp exact)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int d0 = kofs + 32 * kb + 16 * g;  // offset of the group's first key
            const int bidx = min(max(d0 - dlo + PADL, 0), gtop);
            const float* grp = relrow + bidx;
#pragma unroll
            for (int e = 0; e < 8; ++e) rv[kb][8 * g + e] = grp[KSTR * e];
          }
      }
      if (need_mask) {
        finish(rv, std::true_type{});
      } else {
        finish(rv, std::false_type{});
      }
    }
    if constexpr (SHAW && HAS_WV && !GRAPH) {
      // The value term needs the final logit of every key whose label holds
      // that key alone.  Each group of 8 that touches such an offset is stored
      // whole at its own label entries (PADL + delta - dlo onwards).  A lane's
      // offsets grow from tile to tile and all gathers of a tile precede these
      // stores, so the entries overwritten here are never gathered again: the
      // entries a later group reads lie above every offset stored so far, or
      // (fully past the band) in the top SPAN entries of the upper padding,
      // which no store reaches.
      if (!off_band) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int d0 = kofs + 32 * kb + 16 * g;
            if (q_ok && d0 + (SPAN - 1) >= wb_lo && d0 <= wb_hi) {
              float* dst = myLE + (d0 - dlo + PADL);
#pragma unroll
              for (int e = 0; e < 8; ++e) dst[KSTR * e] = s[kb][8 * g + e];
            }
          }
      }
    }

    // online softmax: one cross-lane max per tile, everything else per lane
    tmax = halves_max(tmax);
    const bool grow = tmax > m_run + kRescaleSlack;  // -inf + slack is -inf
    if (__any(grow)) {  // wave-uniform
      const float m_next = grow ? tmax : m_run;
      const float alpha = fast_exp2(m_run - m_next);  // 0 when m_run is -inf
      [[maybe_unused]] const bool had_max = m_run != kNegInf;
      m_run = m_next;
      l_part *= alpha;
      if constexpr (SHAW && HAS_WV) thi *= alpha;
#pragma unroll
      for (int mb = 0; mb < DVB; ++mb) oacc[mb] *= alpha;
      if constexpr (GRAPH && HAS_WV) {
        // the weight sums follow the row's scale (still all zero while the row
        // had no visible key)
        if (grow && had_max)
          for (int r = 0; r < p.nr; ++r) myS[r] *= alpha;
      }
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;

    // the weights; in bf16 also as the operands of the P.V product, whose
    // row sum is taken from those same operands by pairwise dot products with
    // (1, 1), so that the normaliser sums exactly the weights the product uses
    float psum = 0.f;
    [[maybe_unused]] bf16x8 pbw[BF16 ? NKB : 1][2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(s[kb][i] - m_use);
        s[kb][i] = pv;
        if constexpr (BF16) pbw[kb][i >> 3][i & 7] = (__bf16)pv;
        else psum += pv;
      }
    }
    if constexpr (BF16) {
      bf16x2 one;
      one[0] = (__bf16)1.f;
      one[1] = (__bf16)1.f;
      float acc2[2] = {0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            bf16x2 pr;
            pr[0] = pbw[kb][t2][e];
            pr[1] = pbw[kb][t2][e + 1];
            acc2[t2] = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc2[t2], false);
          }
      psum = acc2[0] + acc2[1];
    }
    l_part += psum;
    if constexpr (GRAPH && HAS_WV) {
      // each key's weight into its label's sum, in this lane's own row
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int e = 0; e < 8; ++e) myS[glabel(kb, g, e)] += s[kb][8 * g + e];
    }
    if constexpr (SHAW && HAS_WV && !GRAPH) {
      // +c bucket (keys at offset >= c); empty under the causal mask
      if (!p.causal && !all_lo) {
        if (dmin >= hi_from) {
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
        bf16x4 vlo[2 * DVB], vhi[2 * DVB];
        const uint32_t vt_lds = smem_addr + (uint32_t)(Vt - smem);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb)
            frag_col_issue_blk<ROWB>(2 * kb + t2, vt_lds + trb_lo[mb], vt_lds + trb_hi[mb],
                                     vlo[t2 * DVB + mb], vhi[t2 * DVB + mb]);
        frag_col_wait(vlo, vhi);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb)
            oacc[mb] = mfma(frag_join(vlo[t2 * DVB + mb], vhi[t2 * DVB + mb]), pbw[kb][t2],
                            oacc[mb]);
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) {
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) {
            const int dv = min(32 * mb + ql, D - 1);  // rows past D are never stored
            oacc[mb] = mfma(elem_f32<ROWB>(Vt, 32 * kb + 2 * s2 + hh, dv), s[kb][s2], oacc[mb]);
          }
        }
      }
    }
  }
  for (; t < ntiles; ++t, st_cur = (st_cur + 1 == nstage) ? 0 : st_cur + 1,
                    st_next = (st_next + 1 == nstage) ? 0 : st_next + 1) {
    XrOps xr;
    tile_head(t, st_next, false, xr);
  }
  if (wv_ring && wv_stage < 0) {
    // no tile ran: any stage is free
    wv_stage = 0;
    dma_tile<ROWB, NW>(smem_lds, wvh, p.wv_sr, p.r_lo, r_hi, lay.wv_rows, wave, lane);
  }
  wait_vm<0>();  // the value table has landed
  block_sync();

  // ---- epilogue
  const float l = halves_sum(l_part);
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  if (p.lse && q_ok && hh == 0) {
    // the logits and m_run are in log2 units
    const float m_fin2 = (m_run == kNegInf) ? 0.f : m_run;
    p.lse[b * p.lse_sb + h * p.lse_sh + qi] = l > 0.f ? (m_fin2 + log2f(l)) * kLn2 : kNegInf;
  }
  if constexpr (SHAW && HAS_WV) {
    const float thi_all = halves_sum(thi);
    const float m_fin = (m_run == kNegInf) ? 0.f : m_run;
    // label indices (r - r_lo) whose key is visible and holds the label
    // alone: r in [1, 2c-1], key j = qi + r - c in [0, kv_len), j <= qi if causal
    int r_in_hi = min(2 * c - 1, c - qi + kv_len - 1);
    if (p.causal) r_in_hi = min(r_in_hi, c);
    const int i_in_lo = max(1, c - qi) - p.r_lo;
    const int i_in_hi = q_ok ? r_in_hi - p.r_lo : i_in_lo - 1;
    const bool any_in = i_in_hi >= i_in_lo;
    const unsigned i_in_w = (unsigned)(i_in_hi - i_in_lo);
    const int i_thi = 2 * c - p.r_lo;  // label +c (index past nr when unreachable)
    // label index of this lane's e-th weight in 16-label step ls
    auto label_of = [&](int ls, int e) __attribute__((always_inline)) {
      return BF16 ? ls * 16 + 8 * hh + e : ls * 16 + 2 * e + hh;
    };
    const int nls = (p.nr + 15) / 16;
    const int ls_chunk = lay.wv_chunk / 16;
    int loaded = 0;  // chunk of w^V rows in LDS (chunked staging)
    float isum = 0.f, tlo_all = 0.f;
    // label -c, whose weight is what the row sum leaves after all others, sits
    // in step 0: do that step last
    for (int it = 0; it < nls; ++it) {
      const int ls = (it + 1 < nls) ? it + 1 : 0;
      int lsr = ls;  // step within the staged rows
      int wv_off = lay.wv;
      if (p.wv_mode == kWvChunked) {
        const int ch = ls / ls_chunk;
        if (it == 0 || ch != loaded) {
          block_sync();
          dma_tile<ROWB, NW>(smem_lds, wvh, p.wv_sr, p.r_lo + ch * lay.wv_chunk, r_hi,
                             lay.wv_chunk, wave, lane);
          wait_vm<0>();
          block_sync();
          loaded = ch;
        }
        lsr = ls - ch * ls_chunk;
        wv_off = 0;
      } else if (p.wv_mode == kWvRing) {
        wv_off = wv_stage * G::STAGEB;
      }
      float w[8];
      if constexpr (GRAPH) {
        // graph mode: the two halves' weight sums, already at the row's final
        // scale
        const float* rowS = reinterpret_cast<const float*>(smem + lay.se) + 2 * qrow * lay.ses;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int idx = label_of(ls, e);
          w[e] = (q_ok && idx < p.nr) ? rowS[idx] + rowS[lay.ses + idx] : 0.f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int idx = label_of(ls, e);
          const float x = myLE[PADL + idx];  // inside the row for every step
          const bool ok = any_in && (unsigned)(idx - i_in_lo) <= i_in_w;
          w[e] = ok ? fast_exp2(x - m_fin) : 0.f;
          isum += w[e];
        }
        if (it + 1 == nls) {
          // every single-key weight is in isum now
          tlo_all = fmaxf(l - halves_sum(isum) - thi_all, 0.f);
          if (p.r_lo == 0 && hh == 0) w[0] += tlo_all;  // label index 0 is -c
        }
        if (!p.causal) {
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] += (label_of(ls, e) == i_thi) ? thi_all : 0.f;
        }
        if (!q_ok) {
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = 0.f;
        }
      }
      const unsigned char* wvt = smem + wv_off;
      if constexpr (BF16) {
        bf16x8 bw;
#pragma unroll
        for (int e = 0; e < 8; ++e) bw[e] = (__bf16)w[e];
        bf16x4 wlo[DVB], whi[DVB];
        const uint32_t wv_lds = smem_addr + (uint32_t)wv_off;
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb)
          frag_col_issue<ROWB, D>(wv_lds, lsr * 16, 32 * mb, lane, wlo[mb], whi[mb]);
        frag_col_wait(wlo, whi);
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb) oacc[mb] = mfma(frag_join(wlo[mb], whi[mb]), bw, oacc[mb]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) {
            const int dv = min(32 * mb + ql, D - 1);
            oacc[mb] = mfma(elem_f32<ROWB>(wvt, lsr * 16 + 2 * e + hh, dv), w[e], oacc[mb]);
          }
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

constexpr int kBlockKeys = 64;  // keys per tile, bf16
constexpr int kBlockKeysD128 = 32;  // bf16 d = 128 with two waves per SIMD
constexpr int kBlockKeysF32 = 32;

template <bool BF16, int D, int NW, int BC>
static size_t lds_bytes_t(RelMode mode, bool has_wk, bool has_wv, int nr, int nstage,
                          int t5_dist, int t5_nb, int wv_mode) {
  using G = Geo<BF16, D, NW, BC>;
  const Layout L = make_layout<BF16, D, NW, BC>(mode, has_wk, has_wv, nr, nstage, t5_dist, t5_nb,
                                                wv_mode);
  if ((mode == kRelShaw || mode == kRelGraph) && has_wv && wv_mode == kWvRing &&
      L.wv_rows * G::ROWB > G::STAGEB)
    return ~(size_t)0;  // the w^V tile does not fit one ring stage
  return (size_t)L.total;
}

size_t lds_bytes(bool bf16, int d, const LaunchCfg& cfg, RelMode mode, bool has_wk,
                 bool has_wv, int nr, int t5_dist, int t5_nb) {
#define RELATTN_LDS_CASE(BF, DD, NWW, BCC)                                                 \
  if (bf16 == BF && d == DD && cfg.waves == NWW && cfg.kblock == BCC)                \
    return lds_bytes_t<BF, DD, NWW, BCC>(mode, has_wk, has_wv, nr, cfg.nstage, t5_dist, \
                                         t5_nb, cfg.wv_mode);
#define RELATTN_LDS_D(BF, NWW, BCC) \
  RELATTN_LDS_CASE(BF, 16, NWW, BCC) RELATTN_LDS_CASE(BF, 32, NWW, BCC) \
  RELATTN_LDS_CASE(BF, 64, NWW, BCC) RELATTN_LDS_CASE(BF, 128, NWW, BCC)
  RELATTN_LDS_D(true, 1, kBlockKeys)
  RELATTN_LDS_D(true, 2, kBlockKeys)
  RELATTN_LDS_D(true, 4, kBlockKeys)
  if (bf16 && d == 128 && cfg.kblock == kBlockKeysD128) {
    if (cfg.waves == 2)
      return lds_bytes_t<true, 128, 2, kBlockKeysD128>(mode, has_wk, has_wv, nr, cfg.nstage,
                                                       t5_dist, t5_nb, cfg.wv_mode);
    if (cfg.waves == 4)
      return lds_bytes_t<true, 128, 4, kBlockKeysD128>(mode, has_wk, has_wv, nr, cfg.nstage,
                                                       t5_dist, t5_nb, cfg.wv_mode);
  }
  RELATTN_LDS_D(false, 1, kBlockKeysF32)
  RELATTN_LDS_D(false, 2, kBlockKeysF32)
#undef RELATTN_LDS_D
#undef RELATTN_LDS_CASE
  return ~(size_t)0;  // no such kernel
}

template <int D, int NW, int BC, bool BF16, int MODE, bool HAS_WK, bool HAS_WV>
static int launch_t(const FwdParams& p, void* stream) {
  auto kern = fwd_kernel<D, NW, BC, BF16, MODE, HAS_WK, HAS_WV>;
  const size_t lds = lds_bytes_t<BF16, D, NW, BC>((RelMode)MODE, HAS_WK, HAS_WV, p.nr,
                                                  p.nstage, p.t5_dist, p.t5.nb, p.wv_mode);
  static std::atomic<int> lds_set[64];
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), lds, lds_set);
  if (e != hipSuccess) return (int)e;
  const long long grid = (long long)p.B * p.H * p.n_qtiles;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * NW), lds,
                     reinterpret_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

template <int D, int NW, int BC, bool BF16>
static int launch_mode(RelMode mode, bool has_wk, bool has_wv, const FwdParams& p,
                       void* stream) {
  if (mode == kRelT5) return launch_t<D, NW, BC, BF16, kRelT5, false, false>(p, stream);
  if (mode == kRelGrid) return launch_t<D, NW, BC, BF16, kRelGrid, false, false>(p, stream);
  if (mode == kRelLabel) return launch_t<D, NW, BC, BF16, kRelLabel, false, false>(p, stream);
  if (mode == kRelXL) {
    if constexpr (D <= 64 || BF16) return launch_t<D, NW, BC, BF16, kRelXL, false, false>(p, stream);
    return (int)hipErrorInvalidValue;
  }
  if (mode == kRelGraph) {
    if (has_wk && has_wv) return launch_t<D, NW, BC, BF16, kRelGraph, true, true>(p, stream);
    if (has_wk) return launch_t<D, NW, BC, BF16, kRelGraph, true, false>(p, stream);
    if (has_wv) return launch_t<D, NW, BC, BF16, kRelGraph, false, true>(p, stream);
    return (int)hipErrorInvalidValue;
  }
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
    if (cfg.kblock == kBlockKeysD128 && d == 128) {
      if (cfg.waves == 2)
        return launch_mode<128, 2, kBlockKeysD128, true>(mode, has_wk, has_wv, p, stream);
      if (cfg.waves == 4)
        return launch_mode<128, 4, kBlockKeysD128, true>(mode, has_wk, has_wv, p, stream);
      return (int)hipErrorInvalidValue;
    }
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
