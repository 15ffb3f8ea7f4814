// Lean bf16 forward of relation-aware self-attention for gfx950: the Shaw key
// and value tables, a scalar bias by T5 bucket or by clipped offset, and plain
// attention ("Self-Attention with Relative Position Representations", section
// 3.4, Eq. 3, Eq. 4 and the split of Eq. 5; T5 section of "Relative position
// embeddings").  The same method as the general kernel in relattn_kernels.hip,
// restricted to the hot shapes (bf16, d = 64 or 128, label windows that fit on
// chip) and laid out for the shortest dependency chain per wave:
//
// * Every K/V tile a workgroup reads is requested in the prologue when the
//   ring holds them all (a whole 256-key sequence at d = 64); otherwise the
//   ring streams S - 1 tiles ahead.  Stage loads use per-lane 32-bit offsets
//   computed once, so a request is one address add per instruction.
// * Logits of tiles that lie entirely beyond the clip window take the
//   window's end value, a per-lane constant: their row max is taken on the raw
//   products (one v_max3 per two keys) and the exponent is one fused
//   multiply-add per key, exp2(s * scale + (L_end - m)).
// * Inside the band the relative logits are gathered from one LDS row per
//   query (padding makes the clamped group base exact, and under the causal
//   mask the padding above offset 0 holds -inf, so no per-key causal mask).
// * The value term keeps the in-band logits in the relative row and adds
//   S W^V with MFMA in the epilogue, as the general kernel does.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "relattn_device.h"
#include "relattn_internal.h"
#include "relattn_tiles.h"

namespace relattn {

namespace {

constexpr float kSlack = 8.f;  // log2 units a row max may run ahead of the one in use

typedef float f32x2 __attribute__((ext_vector_type(2)));

// One 16-byte K fragment read from LDS (32-key block kb of the tile at the
// lane's byte address ad), as inline assembly so that all of a tile's reads
// are in flight together; the caller waits with lgkmcnt(0).
template <int ROWB>
__device__ __forceinline__ void kfrag_issue(int kb, uint32_t ad, bf16x8& out) {
  switch (kb) {  // resolved at compile time once the caller's loops unroll
    case 0: asm volatile("ds_read_b128 %0, %1" : "=v"(out) : "v"(ad)); break;
    case 1: asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(out) : "v"(ad), "n"(32 * ROWB)); break;
    case 2: asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(out) : "v"(ad), "n"(64 * ROWB)); break;
    default: asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(out) : "v"(ad), "n"(96 * ROWB)); break;
  }
}

// max over the two lane halves (lanes l and l ^ 32), without the quieting
// of NaN operands that fmaxf needs
__device__ __forceinline__ float halves_max3(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// max(a, b, c) as one v_maximum3_f32 (NaN-propagating maximum needs no quieting
// of its operands, unlike fmaxf; no operand here is ever NaN)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

template <int D, int NW, int BC>
struct LGeo {
  static constexpr int ROWB = 2 * D;                    // bytes per K/V/Q row
  static constexpr int BR = 32 * NW;                    // query rows per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int NKB = BC / 32;                   // 32-key blocks per tile
  static constexpr int NKS = D / 16;                    // MFMA steps over d
  static constexpr int DVB = D / 32;                    // 32-wide blocks of d_v
  static constexpr int TILEB = BC * ROWB;
  static constexpr int STAGEB = 2 * TILEB;              // K tile, then V tile
  static constexpr int SLPW = STAGEB / 1024 / NW;       // stage DMA instructions per wave
  static constexpr int QLPW = BR * ROWB / 1024 / NW;    // Q-tile DMA instructions per wave
  static constexpr int SPAN = 8, PADL = 7, PADU = 15;   // relative-row padding (see below)
  static_assert(STAGEB % (1024 * NW) == 0, "stage must split into whole 1 KB instructions");
  static_assert(BR * ROWB % (1024 * NW) == 0, "Q tile must split into whole 1 KB instructions");
};

// LDS regions of one workgroup, in bytes (host and device).
struct LLayout {
  int q, wk, wv, le, tbc, tb, total;
  int wk_rows, wv_rows, lrs;  // table rows staged; relative-row stride (floats)
};

template <int D, int NW, int BC>
__host__ __device__ inline LLayout lean_layout(int mode, bool has_wk, bool has_wv, int nr,
                                               int nstage, int t5_dist, int t5_nb) {
  using G = LGeo<D, NW, BC>;
  LLayout L{};
  int off = nstage * G::STAGEB;
  auto take = [&](int bytes) {
    const int at = off;
    off += (bytes + 15) & ~15;
    return at;
  };
  const bool shaw = mode == kRelShaw, t5 = mode == kRelT5;
  L.q = take(G::BR * G::ROWB);
  L.wk_rows = dma_rows((nr + 31) & ~31, G::ROWB);
  L.wv_rows = dma_rows((nr + 15) & ~15, G::ROWB);
  L.wk = (shaw && has_wk) ? take(L.wk_rows * G::ROWB) : off;
  L.wv = (shaw && has_wv) ? take(L.wv_rows * G::ROWB) : off;
  // relative row: PADL copies of the first label, the labels, PADU copies of
  // the last (and room for whole 32-label blocks of the relative-key product,
  // whose entries past the last label the padding then overwrites); a stride
  // of 2 mod 4 keeps the lanes' diagonal and column reads nearly free of bank
  // conflicts
  const int m = max(nr + G::PADL + G::PADU, G::PADL + ((nr + 31) & ~31));
  L.lrs = m + ((2 - m) & 3);
  L.le = (shaw && (has_wk || has_wv)) ? take(G::BR * L.lrs * 4) : off;
  L.tbc = t5 ? take(((t5_nb + 63) & ~63) * 4) : off;
  L.tb = t5 ? take((2 * t5_dist + 1 + G::PADL + G::PADU) * 4) : off;
  L.total = off;
  return L;
}

// Waves per SIMD the register budget is sized for (two: 256 registers; the
// tile loop's live values do not fit the 168 of three without spilling).
template <int MODE>
constexpr int lean_waves_per_simd() {
  return 2;
}
template <int D, int NW, int BC, int MODE, bool HAS_WK, bool HAS_WV>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(lean_waves_per_simd<MODE>())))
void fwd_bf16_kernel(const FwdParams p) {
  using G = LGeo<D, NW, BC>;
  using T = __bf16;
  constexpr int NKB = G::NKB, NKS = G::NKS, DVB = G::DVB, ROWB = G::ROWB;
  constexpr int SLPW = G::SLPW, PADL = G::PADL, PADU = G::PADU, SPAN = G::SPAN;
  constexpr int RPI_Q = 1024 / ROWB;  // rows per 1 KB request
  constexpr bool SHAW = MODE == kRelShaw;
  constexpr bool T5 = MODE == kRelT5;
  constexpr bool GATHER = (SHAW && HAS_WK) || T5;  // a relative logit gathered in the band

  // ---- which tile (the dealing of the general kernel; divisions by the
  // host's multiply-high constants)
  auto udiv = [](uint32_t x, uint32_t m, int sh) __attribute__((always_inline)) {
    return (int)((__umulhi(x, m) + x) >> sh);
  };
  int bh, qt;
  const int ng = gridDim.x, nq = p.n_qtiles;
  const int hpx = udiv((uint32_t)(ng >> 3), p.dv_qt_m, p.dv_qt_s);  // heads per XCD
  if (p.causal && (ng & 7) == 0 && hpx * nq == (ng >> 3)) {
    const int x = blockIdx.x & 7, loc = blockIdx.x >> 3;
    const int rank = udiv((uint32_t)loc, p.dv_hpx_m, p.dv_hpx_s);
    bh = x * hpx + (loc - rank * hpx);
    qt = nq - 1 - rank;
  } else {
    const int lid = xcd_remap(blockIdx.x, ng);
    bh = udiv((uint32_t)lid, p.dv_qt_m, p.dv_qt_s);
    qt = lid - bh * nq;
    if (p.causal) qt = nq - 1 - qt;
  }
  const int b = udiv((uint32_t)bh, p.dv_h_m, p.dv_h_s), h = bh - b * p.H;
  const int i0 = qt * G::BR;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const int qrow = wave * 32 + ql;
  const int qi = i0 + qrow;
  const bool q_ok = qi < p.n;
  const int wq0 = i0 + wave * 32;
  const int c = p.clip;
  const int nstage = p.nstage;

  const LLayout lay = lean_layout<D, NW, BC>(MODE, HAS_WK, HAS_WV, p.nr, nstage, p.t5_dist,
                                             p.t5.nb);
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char RELATTN_LDS* smem_lds = (unsigned char RELATTN_LDS*)smem;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem_lds;
  float* myLE = reinterpret_cast<float*>(smem + lay.le) + qrow * lay.lrs;
  float* TBC = reinterpret_cast<float*>(smem + lay.tbc);
  float* TB = reinterpret_cast<float*>(smem + lay.tb);

  const T* qg = reinterpret_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const T* kg = reinterpret_cast<const T*>(p.k) + b * p.k_sb + h * p.k_sh;
  const T* vg = reinterpret_cast<const T*>(p.v) + b * p.v_sb + h * p.v_sh;
  T* og = reinterpret_cast<T*>(p.o) + b * p.o_sb + h * p.o_sh;
  const T* wkh = reinterpret_cast<const T*>(p.wk) + h * p.wk_sh;
  const T* wvh = reinterpret_cast<const T*>(p.wv) + h * p.wv_sh;
  const int r_hi = p.r_lo + p.nr - 1;

  // ---- requests, oldest first: the Q tile, the tables, the first K/V tiles.
  // Query rows past n and key rows past the key length read the last valid
  // row (finite, never stored or counted).
  if (i0 + G::BR <= p.n && (int64_t)RPI_Q * p.q_sn * 2 < ((int64_t)1 << 31)) {
    // every row of the tile exists: instruction I covers rows I*RPI.. (RPI rows
    // of ROWB bytes per 1 KB), lane l row l / CPR, 16-byte chunk l % CPR
    // swizzled by its row.  The swizzle sees row bits 0-3 only, so a lane's
    // byte offset within its instruction's rows takes NV values, by I mod NV.
    constexpr int CPR = ROWB / 16, RPI = 1024 / ROWB;
    constexpr int NV = RPI < 16 ? 16 / RPI : 1;
    const int lrow = lane / CPR, lch = lane % CPR;
    const int64_t rowb = p.q_sn * 2;
    uint32_t lo[NV];
#pragma unroll
    for (int var = 0; var < NV; ++var) {
      const int r = var * RPI + lrow;
      lo[var] = (uint32_t)(lrow * rowb) + (uint32_t)((lch ^ chunk_swizzle<CPR>(r)) * 16);
    }
    const unsigned char* qbase = reinterpret_cast<const unsigned char*>(qg) + (int64_t)i0 * rowb;
#pragma unroll
    for (int k = 0; k < G::QLPW; ++k) {
      const int I = wave + k * NW;
      const unsigned char* src = qbase + (int64_t)I * RPI * rowb;
      uint32_t off = lo[0];
#pragma unroll
      for (int v = 1; v < NV; ++v) off = (I % NV == v) ? lo[v] : off;
      __builtin_amdgcn_global_load_lds((const RELATTN_GLOBAL void*)(src + off),
                                       (RELATTN_LDS void*)(smem_lds + lay.q + I * 1024), 16, 0, 0);
    }
  } else {
    dma_tile<ROWB, NW>(smem_lds + lay.q, qg, p.q_sn, i0, p.n - 1, G::BR, wave, lane);
  }
  compiler_fence();
  if constexpr (SHAW && HAS_WK)
    dma_tile<ROWB, NW>(smem_lds + lay.wk, wkh, p.wk_sr, p.r_lo, r_hi, lay.wk_rows, wave, lane);
  if constexpr (SHAW && HAS_WV)
    dma_tile<ROWB, NW>(smem_lds + lay.wv, wvh, p.wv_sr, p.r_lo, r_hi, lay.wv_rows, wave, lane);
  if constexpr (T5) {
    // the head's bias column (T5) or the window of its row of a table by
    // offset, 4 bytes per lane, by wave 0
    if (wave == 0) {
      for (int I = 0; I * 64 < p.t5.nb; ++I) {
        const int e = min(I * 64 + lane, p.t5.nb - 1) + p.ob_lo;
        __builtin_amdgcn_global_load_lds(
            (const RELATTN_GLOBAL void*)(p.t5_bias + e * p.tb_sb + h * p.tb_sh),
            (RELATTN_LDS void*)(smem_lds + lay.tbc + I * 256), 4, 0, 0);
      }
    }
  }
  compiler_fence();
  // key range (the key length by a scalar load issued after the first
  // requests; the opaque move keeps it from being hoisted above them)
  int kv_len = p.n;
  if (p.key_lens) {
    const int32_t* klp = p.key_lens + b;
    asm volatile("" : "+s"(klp));
    kv_len = min(max(*(const RELATTN_CONST int32_t*)klp, 0), p.n);
  }
  const int kv_end = p.causal ? min(kv_len, i0 + G::BR) : kv_len;
  const int kv_last = max(kv_len - 1, 0);
  const int ntiles = (kv_end + BC - 1) / BC;
  // every tile in the prologue when the ring holds them all, else S - 1 ahead
  const int npre = ntiles <= nstage ? ntiles : nstage - 1;
  uint32_t soff[SLPW];
  if (p.dma32) stage_offsets<ROWB, NW, BC, T>(soff, p.k_sn, p.v_sn, wave, lane);
  auto issue_stage = [&](int tile, int stage) __attribute__((always_inline)) {
    if (p.dma32 && tile * BC + BC - 1 <= kv_last) {
      dma_stage_fast<ROWB, NW, BC>(smem_lds + stage * G::STAGEB, kg + (int64_t)tile * BC * p.k_sn,
                                   vg + (int64_t)tile * BC * p.v_sn, soff, wave);
    } else {
      dma_stage<ROWB, NW, BC>(smem_lds + stage * G::STAGEB, kg, p.k_sn, vg, p.v_sn, tile * BC,
                              kv_last, wave, lane);
    }
    compiler_fence();
  };
  for (int s = 0; s < npre; ++s) issue_stage(s, s);

  // ---- Q as the B operand of S^T = K Q^T, in registers for the whole kernel
  wait_vm_dyn(npre * SLPW);
  block_sync();  // Q, the tables (and the bias column) landed for every wave
  bf16x8 qop[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qop[ks] = frag_row<ROWB>(smem + lay.q, qrow, 2 * ks + hh);

  // ---- relative logits, log2 units.  Shaw: this wave's rows of
  // scale*log2e*q.w^K_r for the reachable labels r_lo.., with PADL copies of
  // the first label below and PADU of the last above.  T5: one shared vector
  // of log2e*bias by offset in [-dist, dist], padded the same way.
  float Llo = 0.f, Lhi = 0.f;
  if constexpr (SHAW && HAS_WK) {
    const int nlb = (p.nr + 31) / 32;
    // lane's fragment of label row ql, chunk 2ks + hh, in the first 32-label
    // block; later blocks lie 32 rows on, which the swizzle does not see
    uint32_t wfo[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      wfo[ks] = smem_addr + (uint32_t)lay.wk + (uint32_t)tile_offset<ROWB>(ql, (2 * ks + hh) * 16);
    // two label blocks per round: every fragment read of the round is in
    // flight before the first product (the row holds whole blocks, so the
    // stores need no per-label test)
    for (int lb = 0; lb < nlb; lb += 2) {
      const bool two = lb + 1 < nlb;  // wave-uniform
      bf16x8 a[2][NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint32_t ad = wfo[ks] + (uint32_t)(lb * 32 * ROWB);
        asm volatile("ds_read_b128 %0, %1" : "=v"(a[0][ks]) : "v"(ad));
        if (two) asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(a[1][ks]) : "v"(ad), "n"(32 * ROWB));
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+v"(a[0][ks]), "+v"(a[1][ks]));
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (u == 1 && !two) break;
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) acc = mfma(a[u][ks], qop[ks], acc);
        // register i of lane half hh holds label (lb+u)*32 + 8(i>>2) + 4hh + (i&3)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          myLE[PADL + (lb + u) * 32 + 8 * (i >> 2) + 4 * hh + (i & 3)] = acc[i] * p.scale_log2;
      }
    }
    compiler_fence();  // the row was written by both halves of the wave
    // both end values in one round trip, then the padding
    Llo = myLE[PADL];
    Lhi = myLE[PADL + p.nr - 1];
    const float edge = hh ? (p.causal ? kNegInf : Lhi) : Llo;
    float* pad = myLE + (hh ? PADL + p.nr : 0);
    const int npad = hh ? PADU : PADL;
#pragma unroll
    for (int x = 0; x < PADU; ++x)
      if (x < npad) pad[x] = edge;
    compiler_fence();
  }
  if constexpr (T5) {
    const int nb = 2 * p.t5_dist + 1 + PADL + PADU;
    for (int x = tid; x < nb; x += G::NT) {
      const int delta = min(max(x - PADL - p.t5_dist, -p.t5_dist), p.t5_dist);
      const int entry = p.ob ? delta + p.t5_dist : t5_bucket(delta, p.t5);
      TB[x] = (p.causal && x - PADL - p.t5_dist > 0) ? kNegInf : kLog2e * TBC[entry];
    }
    block_sync();
    Llo = TB[PADL];
    Lhi = TB[PADL + 2 * p.t5_dist];
  }

  const int dlo = T5 ? -p.t5_dist : p.r_lo - c;  // offset of entry PADL
  const int nwin = T5 ? 2 * p.t5_dist + 1 : p.nr;
  const int gtop = nwin + PADL + PADU - SPAN;      // highest gather base
  const uint32_t relrow_lds =
      smem_addr + (uint32_t)(T5 ? lay.tb : lay.le + qrow * lay.lrs * 4);
  const int band = T5 ? p.t5_dist : c;             // |j - i| >= band: one end value per tile
  // offsets whose label holds a single key (1 <= r <= 2c - 1, reachable)
  const int wb_lo = max(1, p.r_lo) - c, wb_hi = min(2 * c - 1, r_hi) - c;
  const int hi_from = max(c, 1 - c);    // offsets >= hi_from fall in the +c label
  const int hoff = 8 * hh;              // key offset of this lane half
  const float sl2 = p.scale_log2;

  f32x16 oacc[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) oacc[mb] = f32x16{};
  float m_run = kNegInf, l_part = 0.f, thi = 0.f;
  uint32_t trb_lo[DVB], trb_hi[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) frag_col_base<ROWB, D>(32 * mb, lane, trb_lo[mb], trb_hi[mb]);

  // byte offset in a K tile of this lane's fragment for MFMA k-step ks of the
  // first 32-key block (row k_row_of_mfma_row(ql), chunk 2ks + hh, swizzled;
  // later blocks lie 32 rows on, which the swizzle does not see)
  uint32_t kfo[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    kfo[ks] = (uint32_t)tile_offset<ROWB>(k_row_of_mfma_row<true>(ql), (2 * ks + hh) * 16);

  int st_cur = 0;
  for (int t = 0; t < ntiles; ++t, st_cur = (st_cur + 1 == nstage) ? 0 : st_cur + 1) {
    const int j0 = t * BC;
    {
      // tile t landed for this wave: the requests issued after it are the
      // prologue's later tiles, or the stages issued in the loop since
      const int after = (ntiles <= nstage) ? (ntiles - 1 - t)
                                           : min(nstage - 2, ntiles - 1 - t);
      if (after == 0) wait_vm<0>();
      else if (after == 1) wait_vm<SLPW>();
      else wait_vm_dyn(after * SLPW);
    }
    block_sync();  // ... and for every wave; the stage of tile t - 1 is free
    if (ntiles > nstage && t + nstage - 1 < ntiles) {
      const int st_next = (st_cur == 0) ? nstage - 1 : st_cur - 1;
      issue_stage(t + nstage - 1, st_next);
    }
    if (wq0 >= p.n) continue;                 // no live query in this wave
    if (p.causal && j0 > wq0 + 31) continue;  // tile entirely in the future

    const unsigned char* Kt = smem + st_cur * G::STAGEB;
    const unsigned char* Vt = Kt + G::TILEB;

    // S^T block kb: rows = keys j0 + 32kb + .., columns = this wave's queries.
    // Every K fragment of the tile is requested before the first product.
    // (KPF blocks at a time: all of them with the Shaw tables' register
    // budget, one at a time under the tighter one of three waves per SIMD)
    f32x16 s[NKB];
    {
      constexpr int KPF = lean_waves_per_simd<MODE>() == 2 ? NKB : 1;
      const uint32_t kt_lds = smem_addr + (uint32_t)(Kt - smem);
#pragma unroll
      for (int k0 = 0; k0 < NKB; k0 += KPF) {
        bf16x8 a[KPF][NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const uint32_t ad = kt_lds + kfo[ks];
#pragma unroll
          for (int kb = 0; kb < KPF; ++kb) kfrag_issue<ROWB>(k0 + kb, ad, a[kb][ks]);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int kb = 0; kb < KPF; ++kb)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+v"(a[kb][ks]));
#pragma unroll
        for (int kb = 0; kb < KPF; ++kb) {
          s[k0 + kb] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) s[k0 + kb] = mfma(a[kb][ks], qop[ks], s[k0 + kb]);
        }
      }
    }

    // Register (kb, 8g + e) holds key j0 + hoff + 32kb + 16g + e: offset
    // kofs + 32kb + 16g + e from this lane's query.
    const int kofs = j0 + hoff - qi;
    const int dmin = j0 - (wq0 + 31), dmax = j0 + BC - 1 - wq0;
    const bool all_lo = dmax <= -band, all_hi = dmin >= band;  // wave-uniform
    // the band path: a gathered relative logit, or (value table without key
    // table) the band logits the value term keeps
    constexpr bool BANDED = GATHER || (SHAW && HAS_WV);
    const bool off_band = !BANDED || all_lo || all_hi;
    // per-key masking: key-length cuts, and causal cuts that no -inf padding
    // carries (no gathered term, or a tile off the band)
    const bool causal_cut = p.causal && j0 + BC - 1 > wq0;
    const bool need_mask = (j0 + BC > kv_len) || (causal_cut && (off_band || !GATHER));
    const int lim = min(kv_len - 1 - j0 - hoff, p.causal ? -kofs : 0x3fffffff);

    // The rest of the tile, specialised on the two wave-uniform cases: off the
    // band (one relative logit for the whole tile) or in it, and with or
    // without per-key masking.  Each case is its own straight-line code, so no
    // value has to be carried across a join of the four.
    bf16x8 pb[NKB][2];  // the weights as the bf16 operands of P.V
    auto tile_rest = [&](auto off_tag, auto mask_tag) __attribute__((always_inline)) {
      constexpr bool OFF = decltype(off_tag)::value;
      constexpr bool MASK = decltype(mask_tag)::value;
      float tmax = kNegInf;
      float cadd = 0.f;  // off the band: exponent = s * sl2 + cadd
      if constexpr (OFF) {
        // one relative logit for the whole tile: max over the raw products
        cadd = GATHER ? (all_lo ? Llo : Lhi) : 0.f;
        if constexpr (MASK) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int ko = 32 * kb + 16 * (i >> 3) + (i & 7);
              s[kb][i] = (ko <= lim) ? s[kb][i] : kNegInf;
            }
        }
        float mr = kNegInf;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; i += 2) mr = max3f(mr, s[kb][i], s[kb][i + 1]);
        tmax = fmaf(mr, sl2, cadd);  // -inf stays -inf
      } else {
        // band: every relative logit of the tile, 8 entries per group read
        // from one clamped base (the row padding makes the clamp exact); all
        // of the tile's reads are in flight before the first use
        f32x2 gv[NKB][2][4];
        if constexpr (GATHER) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              const int d0 = kofs + 32 * kb + 16 * g;
              const uint32_t ad = relrow_lds + 4u * (uint32_t)min(max(d0 - dlo + PADL, 0), gtop);
              asm volatile("ds_read2_b32 %0, %1 offset1:1" : "=v"(gv[kb][g][0]) : "v"(ad));
              asm volatile("ds_read2_b32 %0, %1 offset0:2 offset1:3" : "=v"(gv[kb][g][1]) : "v"(ad));
              asm volatile("ds_read2_b32 %0, %1 offset0:4 offset1:5" : "=v"(gv[kb][g][2]) : "v"(ad));
              asm volatile("ds_read2_b32 %0, %1 offset0:6 offset1:7" : "=v"(gv[kb][g][3]) : "v"(ad));
            }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
              for (int e2 = 0; e2 < 4; ++e2) asm volatile("" : "+v"(gv[kb][g][e2]));
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              float x = GATHER ? fmaf(s[kb][8 * g + e], sl2, gv[kb][g][e >> 1][e & 1])
                               : s[kb][8 * g + e] * sl2;
              if constexpr (MASK) x = (32 * kb + 16 * g + e <= lim) ? x : kNegInf;
              s[kb][8 * g + e] = x;
            }
          }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; i += 2) tmax = max3f(tmax, s[kb][i], s[kb][i + 1]);
        if constexpr (SHAW && HAS_WV) {
          // the value term needs the final logit of every key whose label
          // holds that key alone: each group of 8 that touches such an offset
          // is stored whole at its own label entries.  A lane's offsets grow
          // from tile to tile and all gathers of a tile precede these stores,
          // so the entries overwritten here are never gathered again (later
          // groups read above every stored offset, or the top SPAN entries of
          // the upper padding, which no store reaches).
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              const int d0 = kofs + 32 * kb + 16 * g;
              if (q_ok && d0 + (SPAN - 1) >= wb_lo && d0 <= wb_hi) {
                float* dst = myLE + (d0 - dlo + PADL);
#pragma unroll
                for (int e = 0; e < 8; ++e) dst[e] = s[kb][8 * g + e];
              }
            }
        }
      }

      // online softmax: one cross-lane max per tile, everything else per lane
      tmax = halves_max3(tmax);
      const bool grow = tmax > m_run + kSlack;  // -inf + slack is -inf
      {
        // rescaled every tile (alpha is exactly 1 while the max in use holds):
        // the multiply is also the move the register allocator wants for the
        // loop-carried accumulators, where a branch taken only on growth costs
        // a copy of all of them on the common path
        const float m_next = grow ? tmax : m_run;
        const float alpha = fast_exp2(m_run - m_next);  // 0 when m_run is -inf
        m_run = m_next;
        l_part *= alpha;
        if constexpr (SHAW && HAS_WV) thi *= alpha;
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb) oacc[mb] *= alpha;
      }
      const float m_use = (m_run == kNegInf) ? 0.f : m_run;
      if constexpr (OFF) {
        const float ca = cadd - m_use;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kb][i] = fast_exp2(fmaf(s[kb][i], sl2, ca));
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kb][i] = fast_exp2(s[kb][i] - m_use);
      }
      // the weights as the bf16 operands of the P.V product, and the row sum
      // of those same operands by pairwise dot products with (1, 1): the
      // normaliser then sums exactly the weights the product used
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[kb][t2][e] = (__bf16)s[kb][8 * t2 + e];
      float psum = 0.f;
      {
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
              pr[0] = pb[kb][t2][e];
              pr[1] = pb[kb][t2][e + 1];
              acc2[t2] = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc2[t2], false);
            }
        psum = acc2[0] + acc2[1];
      }
      l_part += psum;
      if constexpr (SHAW && HAS_WV) {
        // +c label (keys at offset >= c); empty under the causal mask
        if (!p.causal && !all_lo && dmax >= hi_from) {
          if (dmin >= hi_from) {
            thi += psum;
          } else {
            const int hi_ko = hi_from - kofs;  // first key offset in the +c label
            float phi = 0.f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int ko = 32 * kb + 16 * (i >> 3) + (i & 7);
                phi += (ko >= hi_ko) ? s[kb][i] : 0.f;
              }
            thi += phi;
          }
        }
      }

    };
    using Yes = std::true_type;
    using No = std::false_type;
    if (off_band) {
      if (need_mask) tile_rest(Yes{}, Yes{});
      else tile_rest(Yes{}, No{});
    } else {
      if (need_mask) tile_rest(No{}, Yes{});
      else tile_rest(No{}, No{});
    }

    // O^T += V^T P^T (one copy of this code for the four cases above, so the
    // accumulators keep one set of registers through the loop)
    const uint32_t vt_lds = smem_addr + (uint32_t)(Vt - smem);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      bf16x4 vlo[2 * DVB], vhi[2 * DVB];
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
          oacc[mb] = mfma(frag_join(vlo[t2 * DVB + mb], vhi[t2 * DVB + mb]), pb[kb][t2],
                          oacc[mb]);
    }
  }

  // ---- epilogue
  const float l = halves_sum(l_part);
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  if (p.lse && q_ok && hh == 0) {
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
    int i_in_lo = max(1, c - qi) - p.r_lo;
    int i_in_hi = q_ok ? r_in_hi - p.r_lo : i_in_lo - 1;
    // Label +c (its weight is the tail summed in the loop) joins the range as
    // the log of its weight: it is nonzero only when the row has keys at every
    // offset up to c, so its index 2c - r_lo then directly follows the range.
    if (thi_all > 0.f && q_ok) {
      myLE[PADL + 2 * c - p.r_lo] = __builtin_amdgcn_logf(thi_all) + m_fin;
      i_in_hi = 2 * c - p.r_lo;
    }
    if (i_in_hi < i_in_lo) i_in_lo = 1 << 30, i_in_hi = 1 << 30;  // no index passes
    const unsigned i_in_w = (unsigned)(i_in_hi - i_in_lo);
    const int nls = (p.nr + 15) / 16;
    float isum = 0.f;
    const uint32_t wv_lds = smem_addr + (uint32_t)lay.wv;
    // 16 labels per step.  Label -c, whose weight is what the row sum leaves
    // after all others, sits in step 0: that step is taken last.  The steps
    // go up to four at a time (NP of them from it0, all present) with every
    // LDS read of the group in flight before the first exponential.
    auto steps = [&](auto np_tag, int it0) __attribute__((always_inline)) {
      constexpr int NP = decltype(np_tag)::value;
      float x[NP][8];
      bf16x4 wlo[NP][DVB], whi[NP][DVB];
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const int it = it0 + u;
        const int ls = (it + 1 < nls) ? it + 1 : 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[u][e] = myLE[PADL + ls * 16 + 8 * hh + e];  // in the row
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb)
          frag_col_issue<ROWB, D>(wv_lds, ls * 16, 32 * mb, lane, wlo[u][mb], whi[u][mb]);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int u = 0; u < NP; ++u)
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb) asm volatile("" : "+v"(wlo[u][mb]), "+v"(whi[u][mb]));
      float w[NP][8];
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const int it = it0 + u;
        const int ls = (it + 1 < nls) ? it + 1 : 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int idx = ls * 16 + 8 * hh + e;
          const bool ok = (unsigned)(idx - i_in_lo) <= i_in_w;
          // the exponential for every lane, then a select (a conditional
          // exponential becomes a branch per element)
          float ex = fast_exp2(x[u][e] - m_fin);
          asm volatile("" : "+v"(ex));
          w[u][e] = ok ? ex : 0.f;
          isum += w[u][e];
        }
      }
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const int it = it0 + u;
        const int ls = (it + 1 < nls) ? it + 1 : 0;
        if (it + 1 == nls) {
          // every other label's weight is in isum now
          const float tlo_all = fmaxf(l - halves_sum(isum), 0.f);
          if (p.r_lo == 0 && hh == 0 && q_ok) w[u][0] += tlo_all;  // label index 0 is -c
        }
        bf16x8 bw;
#pragma unroll
        for (int e = 0; e < 8; ++e) bw[e] = (__bf16)w[u][e];  // all 0 past the last query
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb)
          oacc[mb] = mfma(frag_join(wlo[u][mb], whi[u][mb]), bw, oacc[mb]);
      }
    };
    int it0 = 0;
    for (; it0 + 4 <= nls; it0 += 4) steps(std::integral_constant<int, 4>{}, it0);
    switch (nls - it0) {
      case 1: steps(std::integral_constant<int, 1>{}, it0); break;
      case 2: steps(std::integral_constant<int, 2>{}, it0); break;
      case 3: steps(std::integral_constant<int, 3>{}, it0); break;
      default: break;
    }
  }

  if (q_ok) {
    T* orow = og + (int64_t)qi * p.o_sn;
#pragma unroll
    for (int mb = 0; mb < DVB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[mb][4 * g + e] * inv_l);
        *reinterpret_cast<bf16x4*>(orow + 32 * mb + 8 * g + 4 * hh) = o4;
      }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

template <int D, int NW, int BC>
size_t lean_lds_t(RelMode mode, bool has_wk, bool has_wv, int nr, int nstage, int t5_dist,
                  int t5_nb) {
  return (size_t)lean_layout<D, NW, BC>(mode, has_wk, has_wv, nr, nstage, t5_dist, t5_nb).total;
}

template <int D, int NW, int BC, int MODE, bool HAS_WK, bool HAS_WV>
int lean_launch_t(const FwdParams& p, void* stream) {
  auto kern = fwd_bf16_kernel<D, NW, BC, MODE, HAS_WK, HAS_WV>;
  const size_t lds = lean_lds_t<D, NW, BC>((RelMode)MODE, HAS_WK, HAS_WV, p.nr, p.nstage,
                                           p.t5_dist, p.t5.nb);
  static std::atomic<int> lds_set[64];
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), lds, lds_set);
  if (e != hipSuccess) return (int)e;
  const long long grid = (long long)p.B * p.H * p.n_qtiles;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * NW), lds,
                     reinterpret_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

template <int D, int NW, int BC>
int lean_launch_mode(RelMode mode, bool has_wk, bool has_wv, const FwdParams& p, void* stream) {
  if (mode == kRelT5) return lean_launch_t<D, NW, BC, kRelT5, false, false>(p, stream);
  if (mode == kRelShaw) {
    if (has_wk && has_wv) return lean_launch_t<D, NW, BC, kRelShaw, true, true>(p, stream);
    if (has_wk) return lean_launch_t<D, NW, BC, kRelShaw, true, false>(p, stream);
    if (has_wv) return lean_launch_t<D, NW, BC, kRelShaw, false, true>(p, stream);
  }
  if (mode == kRelNone) return lean_launch_t<D, NW, BC, kRelNone, false, false>(p, stream);
  return (int)hipErrorInvalidValue;
}

}  // namespace

bool lean_mode_ok(bool bf16, int d, RelMode mode) {
  // the scalar-bias modes keep the general kernel, whose loop fits three waves
  // per SIMD (measured faster on the T5 workload)
  return bf16 && d == 64 && (mode == kRelNone || mode == kRelShaw);
}

size_t lean_lds_bytes(int d, const LaunchCfg& cfg, RelMode mode, bool has_wk, bool has_wv,
                      int nr, int t5_dist, int t5_nb) {
  if (d == 64 && cfg.kblock == 64) {
    if (cfg.waves == 4)
      return lean_lds_t<64, 4, 64>(mode, has_wk, has_wv, nr, cfg.nstage, t5_dist, t5_nb);
    if (cfg.waves == 8)
      return lean_lds_t<64, 8, 64>(mode, has_wk, has_wv, nr, cfg.nstage, t5_dist, t5_nb);
  }
  return ~(size_t)0;
}

int launch_fwd_lean(int d, const LaunchCfg& cfg, RelMode mode, bool has_wk, bool has_wv,
                    const FwdParams& p, void* stream) {
  if (d == 64 && cfg.kblock == 64) {
    if (cfg.waves == 4) return lean_launch_mode<64, 4, 64>(mode, has_wk, has_wv, p, stream);
    if (cfg.waves == 8) return lean_launch_mode<64, 8, 64>(mode, has_wk, has_wv, p, stream);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace relattn
