// LDS tile layout, LDS-DMA copies, MFMA fragment access and cross-lane
// helpers shared by the forward and backward attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

#include "relattn_device.h"

namespace relattn {

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
  // The lane index passes through an opaque register move so that the address
  // arithmetic below stays at the (rare) call site: hoisted out of the tile
  // loop it would hold eight 64-bit addresses live across the loop, which
  // spills to scratch under tight register budgets.
  asm volatile("" : "+v"(lane));
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

// The same stage with a uniform base pointer per tensor and per-lane 32-bit
// byte offsets computed once (stage_offsets): no clamp and no 64-bit address
// arithmetic per tile, so the loads take the scalar-base + vector-offset
// form.  For tiles that lie entirely below the last valid row.
template <int ROWB, int NW, int BC, typename T>
__device__ __forceinline__ void stage_offsets(uint32_t (&off)[2 * BC * ROWB / 1024 / NW],
                                              int64_t k_stride, int64_t v_stride, int wave,
                                              int lane) {
  constexpr int CPR = ROWB / 16;
  constexpr int NI_TILE = BC * ROWB / 1024;
  constexpr int NI = 2 * NI_TILE;
#pragma unroll
  for (int u = 0; u < NI / NW; ++u) {
    const int I = wave + u * NW;
    const bool is_v = I >= NI_TILE;
    const int o = (is_v ? I - NI_TILE : I) * 1024 + lane * 16;
    const int r = o / ROWB;
    const int c = ((o % ROWB) >> 4) ^ chunk_swizzle<CPR>(r);
    off[u] = (uint32_t)((int64_t)r * (is_v ? v_stride : k_stride) * (int64_t)sizeof(T) + c * 16);
  }
}
template <int ROWB, int NW, int BC, typename T>
__device__ __forceinline__ void dma_stage_fast(unsigned char RELATTN_LDS* st, const T* kbase,
                                               const T* vbase,
                                               const uint32_t (&off)[2 * BC * ROWB / 1024 / NW],
                                               int wave) {
  constexpr int NI_TILE = BC * ROWB / 1024;
  constexpr int NI = 2 * NI_TILE;
#pragma unroll
  for (int u = 0; u < NI / NW; ++u) {
    const int I = wave + u * NW;
    const bool is_v = I >= NI_TILE;  // wave-uniform
    const unsigned char* b = reinterpret_cast<const unsigned char*>(is_v ? vbase : kbase);
    __builtin_amdgcn_global_load_lds((const RELATTN_GLOBAL void*)(b + off[u]),
                                     (RELATTN_LDS void*)(st + I * 1024), 16, 0, 0);
  }
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
// Lane part of the two transpose reads for columns dv0.. of a block of rows
// starting at a multiple of 16 (the swizzle depends on row bits 1-3 only, so
// rows 16 apart differ by a constant offset).
template <int ROWB, int D>
__device__ __forceinline__ void frag_col_base(int dv0, int lane, uint32_t& lo, uint32_t& hi) {
  int col = dv0 + (lane & 16) + 4 * (lane & 3);
  if constexpr (D < 32) col = min(col, D - 4);  // columns past D feed rows never stored
  const int row = 8 * (lane >> 5) + ((lane & 15) >> 2);
  lo = (uint32_t)tile_offset<ROWB>(row, col * 2);
  hi = (uint32_t)tile_offset<ROWB>(row + 4, col * 2);
}
// Transpose reads at precomputed lane bases plus a constant row offset.
template <int OFS>
__device__ __forceinline__ void frag_col_issue_at(uint32_t base_lo, uint32_t base_hi,
                                                  bf16x4& lo, bf16x4& hi) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(base_lo), "n"(OFS));
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(base_hi), "n"(OFS));
}
template <int ROWB>
__device__ __forceinline__ void frag_col_issue_blk(int blk16, uint32_t base_lo, uint32_t base_hi,
                                                   bf16x4& lo, bf16x4& hi) {
  switch (blk16) {  // resolved at compile time once the caller's loops unroll
    case 0: frag_col_issue_at<0>(base_lo, base_hi, lo, hi); break;
    case 1: frag_col_issue_at<16 * ROWB>(base_lo, base_hi, lo, hi); break;
    case 2: frag_col_issue_at<32 * ROWB>(base_lo, base_hi, lo, hi); break;
    default: frag_col_issue_at<48 * ROWB>(base_lo, base_hi, lo, hi); break;
  }
}
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
// Elementwise sum of two MFMA operands, rounded once to the operand type.
__device__ __forceinline__ bf16x8 op_add(bf16x8 a, bf16x8 b) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)((float)a[e] + (float)b[e]);
  return r;
}
__device__ __forceinline__ float op_add(float a, float b) { return a + b; }

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
// which share K and V) run on the same XCD and hence share its L2.  (Causal
// grids whose heads divide evenly over the XCDs use the heaviest-first dealing
// in the kernel instead.)
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int per = G / 8, rem = G % 8, xcd = bid % 8, loc = bid / 8;
  return (xcd < rem) ? xcd * (per + 1) + loc
                     : rem * (per + 1) + (xcd - rem) * per + loc;
}

// Sum and max of a value over the two lane halves (lanes l and l ^ 32, which
// hold the two key halves of the same query): one v_permlane32_swap.
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Host: allow a kernel `lds` bytes of dynamic LDS (needed above 64 KB), at most
// once per kernel, device and size: `done` (one per kernel) remembers the
// largest size set on each device, so repeated launches skip the runtime call.
inline hipError_t allow_dynamic_lds(const void* kern, size_t lds, std::atomic<int> (&done)[64]) {
  if (lds <= 64 * 1024) return hipSuccess;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
  if (dev >= 0 && done[dev].load(std::memory_order_relaxed) >= (int)lds) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess && dev >= 0) {
    int seen = done[dev].load(std::memory_order_relaxed);
    while (seen < (int)lds && !done[dev].compare_exchange_weak(seen, (int)lds)) {
    }
  }
  return e;
}

}  // namespace relattn
