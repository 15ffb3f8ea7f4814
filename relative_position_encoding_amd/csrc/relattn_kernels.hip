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
#include <hip/hip_runtime.h>

#include <type_traits>

#include "relattn_internal.h"

namespace relattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

#define RELATTN_LDS __attribute__((address_space(3)))
#define RELATTN_GLOBAL __attribute__((address_space(1)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// 2^x with the hardware exponential (about 1 ulp; results below 2^-126,
// which cannot change a softmax sum at fp32 precision, flush to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A row max may run ahead of the max used for the exponentials by this much
// (log2 units) before the running sums are rescaled: p <= 2^8 stays exact in
// fp32 sums and in bf16 operands, and most tiles then skip the rescale.
constexpr float kRescaleSlack = 8.f;

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

// ---------------------------------------------------------------------------
// Synchronisation.  The K/V ring is filled by LDS-DMA, which the compiler's
// workgroup fences would drain completely (vmcnt(0)) at every barrier; the
// kernel therefore waits for exactly the tiles it needs with explicit vmcnt
// counts and uses a bare barrier that only orders LDS traffic.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void block_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// vmcnt wait for a count known only at run time (larger counts wait for 0,
// which is never too little)
__device__ __forceinline__ void wait_vm_dyn(int n) {
  switch (n) {
#define RELATTN_VMCASE(k) \
  case k:                 \
    wait_vm<k>();         \
    return;
    RELATTN_VMCASE(1) RELATTN_VMCASE(2) RELATTN_VMCASE(3) RELATTN_VMCASE(4)
    RELATTN_VMCASE(5) RELATTN_VMCASE(6) RELATTN_VMCASE(7) RELATTN_VMCASE(8)
    RELATTN_VMCASE(9) RELATTN_VMCASE(10) RELATTN_VMCASE(11) RELATTN_VMCASE(12)
    RELATTN_VMCASE(13) RELATTN_VMCASE(14) RELATTN_VMCASE(15) RELATTN_VMCASE(16)
    RELATTN_VMCASE(17) RELATTN_VMCASE(18) RELATTN_VMCASE(19) RELATTN_VMCASE(20)
    RELATTN_VMCASE(21) RELATTN_VMCASE(22) RELATTN_VMCASE(23) RELATTN_VMCASE(24)
    RELATTN_VMCASE(25) RELATTN_VMCASE(26) RELATTN_VMCASE(27) RELATTN_VMCASE(28)
    RELATTN_VMCASE(29) RELATTN_VMCASE(30) RELATTN_VMCASE(31) RELATTN_VMCASE(32)
    RELATTN_VMCASE(33) RELATTN_VMCASE(34) RELATTN_VMCASE(35) RELATTN_VMCASE(36)
    RELATTN_VMCASE(37) RELATTN_VMCASE(38) RELATTN_VMCASE(39) RELATTN_VMCASE(40)
    RELATTN_VMCASE(41) RELATTN_VMCASE(42) RELATTN_VMCASE(43) RELATTN_VMCASE(44)
    RELATTN_VMCASE(45) RELATTN_VMCASE(46) RELATTN_VMCASE(47) RELATTN_VMCASE(48)
#undef RELATTN_VMCASE
    default:
      wait_vm<0>();
      return;
  }
}

// ---------------------------------------------------------------------------
// Tile layout in LDS: rows of ROWB bytes, 16-byte chunks XOR-swizzled per row.
// The swizzles were chosen (by enumerating the bank mapping of the fragment
// reads) so that the 16 lanes of a 128-bit read and the 32 lanes of a
// transpose read never share a bank.
// ---------------------------------------------------------------------------
template <int CPR>  // 16-byte chunks per row (power of two)
__host__ __device__ __forceinline__ int chunk_swizzle(int row) {
  if constexpr (CPR >= 16) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return ((((row >> 1) & 1) << 2) | (((row >> 3) & 1) << 1) | ((row >> 2) & 1)) & (CPR - 1);
  }
}
template <int ROWB>
__device__ __forceinline__ int tile_offset(int row, int byte_in_row) {
  constexpr int CPR = ROWB / 16;
  const int chunk = ((byte_in_row >> 4) ^ chunk_swizzle<CPR>(row)) & (CPR - 1);
  return row * ROWB + chunk * 16 + (byte_in_row & 15);
}

// Rows of a DMA'd tile come in whole 1 KB wave instructions.
__host__ __device__ inline int dma_rows(int rows, int rowb) {
  const int g = rowb >= 1024 ? 1 : 1024 / rowb;
  return (rows + g - 1) / g * g;
}

// Copy `rows` rows (a multiple of 1024/ROWB) of a row-major global matrix into
// a swizzled LDS tile.  Row r of the tile reads global row min(row0 + r,
// row_max).  The 1 KB instructions are dealt to the waves round robin; returns
// the number this wave issued.
template <int ROWB, int NW, typename T>
__device__ __forceinline__ int dma_tile(unsigned char RELATTN_LDS* lds, const T* g,
                                        int64_t row_stride, int row0, int row_max, int rows,
                                        int wave, int lane) {
  constexpr int CPR = ROWB / 16;
  const int ninstr = rows * ROWB / 1024;
  int issued = 0;
  for (int I = wave; I < ninstr; I += NW) {
    const int o = I * 1024 + lane * 16;
    const int r = o / ROWB;
    const int c = ((o % ROWB) >> 4) ^ chunk_swizzle<CPR>(r);
    const int grow = min(row0 + r, row_max);
    const T* src = g + (int64_t)grow * row_stride + c * (16 / (int)sizeof(T));
    __builtin_amdgcn_global_load_lds((const RELATTN_GLOBAL void*)src,
                                     (RELATTN_LDS void*)(lds + I * 1024), 16, 0, 0);
    ++issued;
  }
  return issued;
}

// One K/V stage: BC rows of K then BC rows of V, dealt to the waves as one
// sequence of 1 KB instructions so that every wave issues exactly the same
// number per stage (the per-tile vmcnt waits rely on it).
template <int ROWB, int NW, int BC, typename T>
__device__ __forceinline__ void dma_stage(unsigned char RELATTN_LDS* st, const T* kg,
                                          int64_t k_stride, const T* vg, int64_t v_stride,
                                          int row0, int row_max, int wave, int lane) {
  constexpr int CPR = ROWB / 16;
  constexpr int NI_TILE = BC * ROWB / 1024;
  constexpr int NI = 2 * NI_TILE;
  static_assert(NI % NW == 0, "stage must split evenly over the waves");
#pragma unroll
  for (int u = 0; u < NI / NW; ++u) {
    const int I = wave + u * NW;     // instruction within the stage
    const bool is_v = I >= NI_TILE;  // wave-uniform
    const int o = (is_v ? I - NI_TILE : I) * 1024 + lane * 16;
    const int r = o / ROWB;
    const int c = ((o % ROWB) >> 4) ^ chunk_swizzle<CPR>(r);
    const int grow = min(row0 + r, row_max);
    const T* src = (is_v ? vg : kg) + (int64_t)grow * (is_v ? v_stride : k_stride) +
                   c * (16 / (int)sizeof(T));
    __builtin_amdgcn_global_load_lds((const RELATTN_GLOBAL void*)src,
                                     (RELATTN_LDS void*)(st + I * 1024), 16, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Geometry and LDS budget, identical on host and device.
// ---------------------------------------------------------------------------

// Relative-logit rows hold the nr reachable labels between rel_pad copies of
// the first and of the last label on each side: a group of 8 logits (keys
// KSTR apart) then reads 8 entries from one clamped base, whether the group
// lies in the band, in a tail or across an edge.
template <bool BF16>
__host__ __device__ constexpr int rel_pad() { return BF16 ? 8 : 16; }

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
  static constexpr int PAD = rel_pad<BF16>();
  static_assert(STAGEB % (1024 * NW) == 0, "stage must split into whole 1 KB instructions");
};

struct Layout {
  int wk, wv, le, tbc, tb, total;  // byte offsets / total bytes
  int wk_rows, wv_rows, lrs;       // tile rows, relative-row stride (floats)
  int wk_chunk;                    // w^K rows staged at a time (multiple of 32)
  int wv_chunk;                    // w^V rows staged at a time (multiple of 16)
};

// wv_resident: the w^V tile gets its own region, loaded in the prologue;
// otherwise it is staged in chunks through the free ring after the loop.
template <bool BF16, int D, int NW, int BC>
__host__ __device__ inline Layout make_layout(int mode, bool has_wk, bool has_wv, int nr,
                                              int nstage, int t5_dist, int t5_nb,
                                              bool wv_resident) {
  using G = Geo<BF16, D, NW, BC>;
  Layout L{};
  int off = nstage * G::STAGEB;
  auto take = [&](int bytes) {
    const int at = off;
    off += (bytes + 15) & ~15;
    return at;
  };
  const bool shaw = mode == kRelShaw, t5 = mode == kRelT5;
  L.wk_rows = dma_rows((nr + 31) & ~31, G::ROWB);
  L.wv_rows = dma_rows((nr + 15) & ~15, G::ROWB);
  // relative row: padding, nr labels, padding, one dummy slot; even stride so
  // that the rows of one wave hit distinct banks along a diagonal j - i
  L.lrs = (nr + 2 * G::PAD + 1 + 1) & ~1;
  // the w^K tile is read once, before the loop, in label blocks of 32: it is
  // staged in the last ring stage, which receives its first K/V tile only
  // inside the loop (in several chunks if it does not fit)
  L.wk = (nstage - 1) * G::STAGEB;
  L.wk_chunk = min(L.wk_rows, (G::STAGEB / G::ROWB) / 32 * 32);
  if (shaw && has_wv && wv_resident) {
    L.wv = take(L.wv_rows * G::ROWB);
    L.wv_chunk = L.wv_rows;
  } else {
    L.wv = 0;  // ring stages, free after the loop
    L.wv_chunk = min(L.wv_rows, (nstage * G::STAGEB / G::ROWB) / 16 * 16);
  }
  L.le = (shaw && (has_wk || has_wv)) ? take(G::BR * L.lrs * 4) : off;
  L.tbc = t5 ? take(((t5_nb + 63) & ~63) * 4) : off;
  L.tb = t5 ? take((2 * t5_dist + 1 + 2 * G::PAD) * 4) : off;
  L.total = off;
  return L;
}

// Row of the K tile that feeds MFMA row m of a 32-key block.  The order is
// chosen so that accumulator register i of lane half h ends up holding key
// 16(i >> 3) + 8h + (i & 7) (bf16) or 2i + h (fp32), which makes each lane's
// P values a ready MFMA operand for the P.V product.
template <bool BF16>
__device__ __forceinline__ int k_row_of_mfma_row(int m) {
  if constexpr (BF16) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);  // swap bits 2 and 3
  } else {
    return (m & ~7) | ((m & 3) << 1) | ((m >> 2) & 1);
  }
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 8 consecutive bf16 of row `row` starting at column 8 * chunk of a tile
template <int ROWB>
__device__ __forceinline__ bf16x8 frag_row(const unsigned char* tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(tile + tile_offset<ROWB>(row, chunk * 16));
}
// fp32 element (row, col) of a tile
template <int ROWB>
__device__ __forceinline__ float elem_f32(const unsigned char* tile, int row, int col) {
  return *reinterpret_cast<const float*>(tile + tile_offset<ROWB>(row, col * 4));
}
// MFMA A operand of a transposed product from a row-major bf16 tile: lane l
// receives column dv0 + (l & 31) of rows row0 + 8 * (l >> 5) + 0..7.  Two
// transpose reads of 4 rows each; within a 16-lane group, output lane i,
// element k comes from source lane 4k + i/4, element i % 4.
//
// The reads are issued as inline assembly: the compiler cannot tell them
// apart from the K/V stages still streaming into other ring slots by LDS-DMA
// and would otherwise wait for all of those first.  frag_col_wait() completes
// them; its register operands order every use after the wait.
template <int ROWB, int D>
__device__ __forceinline__ void frag_col_issue(uint32_t tile_lds, int row0, int dv0, int lane,
                                               bf16x4& lo, bf16x4& hi) {
  int col = dv0 + (lane & 16) + 4 * (lane & 3);
  if constexpr (D < 32) col = min(col, D - 4);  // columns past D feed rows never stored
  const int row = row0 + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const uint32_t a0 = tile_lds + tile_offset<ROWB>(row, col * 2);
  const uint32_t a1 = tile_lds + tile_offset<ROWB>(row + 4, col * 2);
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(a0));
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(hi) : "v"(a1));
}
__device__ __forceinline__ bf16x8 frag_join(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <int N>
__device__ __forceinline__ void frag_col_wait(bf16x4 (&lo)[N], bf16x4 (&hi)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(lo[i]), "+v"(hi[i]));
}

// Workgroup id -> logical tile id.  Workgroups are dealt to the 8 XCDs round
// robin; this makes consecutive logical ids (tiles of the same batch and head,
// which share K and V) run on the same XCD and hence share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int per = G / 8, rem = G % 8, xcd = bid % 8, loc = bid / 8;
  return (xcd < rem) ? xcd * (per + 1) + loc
                     : rem * (per + 1) + (xcd - rem) * per + loc;
}

// Two waves per SIMD for d <= 64 (they hide each other's softmax and memory
// latency); d = 128 needs the whole register file for one.
template <int D, int NW, int BC, bool BF16, int MODE, bool HAS_WK, bool HAS_WV>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(D <= 64 ? 2 : 1))) void fwd_kernel(const FwdParams p) {
  using G = Geo<BF16, D, NW, BC>;
  using T = typename G::T;
  using Op = std::conditional_t<BF16, bf16x8, float>;
  constexpr int NT = G::NT, NKB = G::NKB, DVB = G::DVB;
  constexpr int NKS = G::NKS, ROWB = G::ROWB, PAD = G::PAD, LPW = G::LPW;
  constexpr bool SHAW = (MODE == kRelShaw);
  constexpr bool T5 = (MODE == kRelT5);
  constexpr bool GATHER = (SHAW && HAS_WK) || T5;  // a gathered relative logit
  constexpr int KSTR = BF16 ? 1 : 2;  // key step between consecutive registers
  constexpr int SPAN = 7 * KSTR + 1;  // keys spanned by a group of 8 registers

  // ---- which tile
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / p.n_qtiles;
  int qt = lid - bh * p.n_qtiles;
  if (p.causal) qt = p.n_qtiles - 1 - qt;  // longest causal rows first
  const int b = bh / p.H, h = bh - b * p.H;
  const int i0 = qt * (32 * NW);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, hh = lane >> 5;
  const int qrow = wave * 32 + ql;
  const int qi = i0 + qrow;
  const bool q_ok = qi < p.n;
  const int wq0 = i0 + wave * 32;
  int kv_len = p.n;
  if (p.key_lens) kv_len = min(max(p.key_lens[b], 0), p.n);
  const int kv_end = p.causal ? min(kv_len, i0 + 32 * NW) : kv_len;
  const int kv_last = max(kv_len - 1, 0);
  const int c = p.clip;
  const int r_hi = p.r_lo + p.nr - 1;
  const int ntiles = (kv_end + BC - 1) / BC;
  const int nstage = p.nstage;

  const Layout lay = make_layout<BF16, D, NW, BC>(MODE, HAS_WK, HAS_WV, p.nr, nstage, p.t5_dist,
                                                  p.t5.nb, p.wv_resident != 0);
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

  // ---- Q as the B operand of S^T = K Q^T, resident for the whole kernel.
  // Rows past n load row n-1 (never stored).
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

  // ---- LDS-DMA, oldest first: relative tables, then the first K/V stages.
  // Key rows past the key length read the last visible row (finite, masked).
  compiler_fence();
  const T* wkh = reinterpret_cast<const T*>(p.wk) + h * p.wk_sh;
  const T* wvh = reinterpret_cast<const T*>(p.wv) + h * p.wv_sh;
  if constexpr (SHAW && HAS_WK) {
    dma_tile<ROWB, NW>(smem_lds + lay.wk, wkh, p.wk_sr, p.r_lo, r_hi, lay.wk_chunk, wave, lane);
  }
  compiler_fence();
  int n_after_wk = 0;  // this wave's DMA instructions issued after the w^K chunk
  if constexpr (SHAW && HAS_WV) {
    if (p.wv_resident)
      n_after_wk += dma_tile<ROWB, NW>(smem_lds + lay.wv, wvh, p.wv_sr, p.r_lo, r_hi,
                                       lay.wv_rows, wave, lane);
  }
  if constexpr (T5) {
    // bias column of this head, 4 bytes per lane, issued by wave 0
    if (wave == 0) {
      for (int I = 0; I * 64 < p.t5.nb; ++I) {
        const int bucket = min(I * 64 + lane, p.t5.nb - 1);
        __builtin_amdgcn_global_load_lds(
            (const RELATTN_GLOBAL void*)(p.t5_bias + bucket * p.tb_sb + h * p.tb_sh),
            (RELATTN_LDS void*)(smem_lds + lay.tbc + I * 256), 4, 0, 0);
      }
    }
  }
  compiler_fence();
  auto issue_stage = [&](int tile) __attribute__((always_inline)) {
    dma_stage<ROWB, NW, BC>(smem_lds + (tile % nstage) * G::STAGEB, kg, p.k_sn, vg, p.v_sn,
                            tile * BC, kv_last, wave, lane);
    compiler_fence();
  };
  const int n_pre = min(nstage - 1, ntiles);
  for (int s = 0; s < n_pre; ++s) issue_stage(s);
  n_after_wk += n_pre * LPW;

  // ---- relative logits in LDS.  Shaw: row qrow holds scale*log2e*q.w^K_r for
  // the reachable label rows r_lo..r_hi at entries PAD + (r - r_lo), padded.
  // T5: one shared vector holds log2e*bias[beta(delta), h] for delta in
  // [-dist, dist] at entries PAD + dist + delta, padded.
  if constexpr (GATHER) {
    wait_vm_dyn(T5 ? n_pre * LPW : n_after_wk);  // the tables are older than the stages
    block_sync();
  }
  if constexpr (SHAW && HAS_WK) {
    const unsigned char* wkt = smem + lay.wk;
    const int nlb = (p.nr + 31) / 32;
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
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        Op a;
        if constexpr (BF16) {
          a = frag_row<ROWB>(wkt, row, 2 * ks + hh);
        } else {
          a = elem_f32<ROWB>(wkt, row, 2 * ks + hh);
        }
        acc = mfma(a, qop[ks], acc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int idx = lb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (idx < p.nr) myLE[PAD + idx] = acc[i] * p.scale_log2;
      }
    }
    compiler_fence();  // the row was written by both halves of this wave
    const float edge = myLE[hh ? PAD + p.nr - 1 : PAD];
    float* pad = myLE + (hh ? PAD + p.nr : 0);
#pragma unroll
    for (int x = 0; x < PAD; ++x) pad[x] = edge;
    compiler_fence();
  }
  if constexpr (T5) {
    const int nb = 2 * p.t5_dist + 1 + 2 * PAD;
    for (int x = tid; x < nb; x += NT) {
      const int delta = min(max(x - PAD - p.t5_dist, -p.t5_dist), p.t5_dist);
      TB[x] = kLog2e * TBC[t5_bucket(delta, p.t5)];
    }
    block_sync();
  }

  // window of offsets delta = j - i covered by the relative row, and the
  // relative logit of its two ends (used for tiles entirely outside the band)
  const int dlo = T5 ? -p.t5_dist : p.r_lo - c;  // delta of entry PAD
  const int nwin = T5 ? 2 * p.t5_dist + 1 : p.nr;
  const float* relrow = T5 ? TB : myLE;
  float Llo = 0.f, Lhi = 0.f;
  if constexpr (GATHER) {
    Llo = relrow[PAD];
    Lhi = relrow[PAD + nwin - 1];
  }
  const int band = T5 ? p.t5_dist : c;  // |j - i| >= band: one end value for the tile

  // ---- running state (per lane: one query, half of each tile's keys)
  f32x16 oacc[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) oacc[mb] = f32x16{};
  float m_run = kNegInf;
  float l_part = 0.f, thi = 0.f;
  const int hi_from = max(c, 1 - c);    // offsets >= hi_from fall in the +c bucket
  const int hoff = BF16 ? 8 * hh : hh;  // key offset of this lane half

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * BC;
    // tile t landed for this wave (the next stage may still be in flight) ...
    if (nstage > 2 && t + 1 < ntiles) {
      wait_vm<LPW>();
    } else {
      wait_vm<0>();
    }
    block_sync();  // ... and for every wave; stage (t - 1) % nstage is free
    if (t + nstage - 1 < ntiles) issue_stage(t + nstage - 1);

    if (wq0 >= p.n) continue;                  // no live query in this wave
    if (p.causal && j0 > wq0 + 31) continue;   // tile entirely in the future

    const unsigned char* Kt = smem + (t % nstage) * G::STAGEB;
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

    // Register (kb, 8g + e) holds key j0 + hoff + 32kb + 16g + KSTR*e, i.e.
    // offset delta = kofs + 32kb + 16g + KSTR*e from this lane's query.
    const int kofs = j0 + hoff - qi;
    const bool need_mask = (j0 + BC > kv_len) || (p.causal && j0 + BC - 1 > wq0);
    // visible iff its key offset within the lane's keys is <= lim
    const int lim = min(kv_len - 1 - j0 - hoff, p.causal ? -kofs : 0x3fffffff);
    const int dmin = j0 - (wq0 + 31), dmax = j0 + BC - 1 - wq0;
    const bool all_lo = dmax <= -band, all_hi = dmin >= band;  // wave-uniform
    const bool off_band = (SHAW || T5) && (all_lo || all_hi);
    // in-band logits go to their own label entry of the relative row (the
    // value term needs them once the row max is final): each such entry is
    // gathered only for its own key, before this write; everything else goes
    // to the dummy entry.  In band: 1 - c <= delta <= c - 1, visible, live row.
    const int sbase = kofs - dlo + PAD;  // entry of key offset 0
    const int lo_ko = 1 - c - kofs;
    const int hi_ko = q_ok ? min(c - 1 - kofs, lim) : lo_ko - 1;
    const unsigned in_width = (unsigned)(hi_ko - lo_ko);
    const bool any_in = hi_ko >= lo_ko;
    const int dummy = p.nr + 2 * PAD;
    float tmax = kNegInf;
    if (!GATHER || off_band) {
      // no gathered term here: nothing relative, the tile's end value, or no
      // key table (then only the value term needs the band logits)
      const float rel = GATHER ? (all_lo ? Llo : Lhi) : 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ko = 32 * kb + 16 * (i >> 3) + KSTR * (i & 7);
          float x = fmaf(s[kb][i], p.scale_log2, rel);
          if constexpr (SHAW && HAS_WV && !HAS_WK) {
            if (!off_band) {
              const bool in = any_in && (unsigned)(ko - lo_ko) <= in_width;
              myLE[in ? sbase + ko : dummy] = x;
            }
          }
          if (need_mask) x = (ko <= lim) ? x : kNegInf;
          s[kb][i] = x;
          tmax = fmaxf(tmax, x);
        }
    } else {
      // band: gather every relative logit of the tile first (8 entries per
      // group from one clamped base, see rel_pad), then combine
      float rv[NKB][16];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int d0 = kofs + 32 * kb + 16 * g;  // offset of the group's first key
          const int bidx = min(max(d0 - dlo + PAD, 0), nwin + 2 * PAD - SPAN);
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
          rv[kb][i] = x;  // unmasked logits of the band, for the value term
          if (need_mask) x = (ko <= lim) ? x : kNegInf;
          s[kb][i] = x;
          tmax = fmaxf(tmax, x);
        }
      if constexpr (SHAW && HAS_WV) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ko = 32 * kb + 16 * (i >> 3) + KSTR * (i & 7);
            const bool in = any_in && (unsigned)(ko - lo_ko) <= in_width;
            myLE[in ? sbase + ko : dummy] = rv[kb][i];
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
            frag_col_issue<ROWB, D>(vt_lds, 32 * kb + 16 * t2, 32 * mb, lane, vlo[t2 * DVB + mb],
                                    vhi[t2 * DVB + mb]);
        bf16x8 pb[2];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[t2][e] = (__bf16)s[kb][8 * t2 + e];
        frag_col_wait(vlo, vhi);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb)
            oacc[mb] = mfma(frag_join(vlo[t2 * DVB + mb], vhi[t2 * DVB + mb]), pb[t2], oacc[mb]);
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
  wait_vm<0>();  // the value table has landed even when no tile ran
  block_sync();

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
      const float e = myLE[PAD + min(idx, p.nr - 1)];
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
    const int nls = (p.nr + 15) / 16;
    const int ls_chunk = lay.wv_chunk / 16;
    for (int ls = 0; ls < nls; ++ls) {
      if (!p.wv_resident && ls % ls_chunk == 0) {
        // stage the next chunk of w^V rows in the (now free) ring
        block_sync();
        dma_tile<ROWB, NW>(smem_lds, wvh, p.wv_sr, p.r_lo + ls * 16, r_hi, lay.wv_chunk, wave,
                           lane);
        wait_vm<0>();
        block_sync();
      }
      const int lsr = ls % ls_chunk;  // label step within the staged chunk
      const unsigned char* wvt = smem + lay.wv;
      if constexpr (BF16) {
        bf16x8 bw;
#pragma unroll
        for (int e = 0; e < 8; ++e) bw[e] = (__bf16)bucket_weight(ls * 16 + 8 * hh + e);
        bf16x4 wlo[DVB], whi[DVB];
        const uint32_t wv_lds = smem_addr + (uint32_t)lay.wv;
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb)
          frag_col_issue<ROWB, D>(wv_lds, lsr * 16, 32 * mb, lane, wlo[mb], whi[mb]);
        frag_col_wait(wlo, whi);
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb) oacc[mb] = mfma(frag_join(wlo[mb], whi[mb]), bw, oacc[mb]);
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          const int idx = ls * 16 + 2 * s2 + hh;
          const float bw = bucket_weight(idx);
#pragma unroll
          for (int mb = 0; mb < DVB; ++mb) {
            const int dv = min(32 * mb + ql, D - 1);
            oacc[mb] = mfma(elem_f32<ROWB>(wvt, lsr * 16 + 2 * s2 + hh, dv), bw, oacc[mb]);
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
constexpr int kBlockKeysF32 = 32;

template <bool BF16, int D, int NW, int BC>
static size_t lds_bytes_t(RelMode mode, bool has_wk, bool has_wv, int nr, int nstage,
                          int t5_dist, int t5_nb, bool wv_resident) {
  return (size_t)make_layout<BF16, D, NW, BC>(mode, has_wk, has_wv, nr, nstage, t5_dist, t5_nb,
                                              wv_resident)
      .total;
}

size_t lds_bytes(bool bf16, int d, const LaunchCfg& cfg, RelMode mode, bool has_wk,
                 bool has_wv, int nr, int t5_dist, int t5_nb) {
#define RELATTN_LDS(BF, DD, NWW, BCC)                                                 \
  if (bf16 == BF && d == DD && cfg.waves == NWW && cfg.kblock == BCC)                \
    return lds_bytes_t<BF, DD, NWW, BCC>(mode, has_wk, has_wv, nr, cfg.nstage, t5_dist, \
                                         t5_nb, cfg.wv_resident);
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
  const size_t lds = lds_bytes_t<BF16, D, NW, BC>((RelMode)MODE, HAS_WK, HAS_WV, p.nr,
                                                  p.nstage, p.t5_dist, p.t5.nb,
                                                  p.wv_resident != 0);
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
