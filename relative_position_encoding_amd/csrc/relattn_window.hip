// Small-window attention with the 2-D relative position bias (survey page
// "Relative position embeddings", Swin paragraph: the T5 scalar bias ported to
// an M x M grid, the table indexed by the flattened 2-D offset), for windows of
// at most 64 tokens, bf16, d = 32 or 64:
//
//   e_ij = scale * q_i . k_j + bias[h', (y_j - y_i + M - 1)(2M - 1) + (x_j - x_i + M - 1)]
//
// with token p at (y, x) = (p / M, p % M), raster order.  The same method as
// the grid mode of the general kernel; what differs is the data flow.  A whole
// window fits one key tile, so each (window, head) is a small independent item
// whose time is mostly memory latency.  The kernel is persistent: a workgroup
// of two waves (query rows 0-31 and 32-63) walks a contiguous run of items of
// one head through a ring of S LDS slots (Q, K and V of one item each), with
// the next S - 1 items requested while the current one is computed, so that
// enough bytes are in flight per compute unit to cover the memory latency.
// Each lane holds the head's bias for its query row and its 32 keys in
// registers (log2 units, -inf for keys and rows past n), built once per head
// from the table staged in LDS, so a logit costs one fused multiply-add.  With
// one key tile the softmax needs no running rescale: one max, one pass of
// exponentials.
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "relattn_device.h"
#include "relattn_internal.h"
#include "relattn_tiles.h"

namespace relattn {

namespace {

constexpr int kWinRows = 64;   // tokens per window at most (one 64-row tile)
constexpr int kWinWaves = 2;
constexpr int kWinThreads = 64 * kWinWaves;

template <int D>
struct WinGeo {
  static constexpr int ROWB = 2 * D;                 // bytes per row
  static constexpr int TILEB = kWinRows * ROWB;      // one 64-row tensor tile
  static constexpr int SLOTB = 3 * TILEB;            // Q, K, V
  static constexpr int S = 3;  // ring slots (measured: 2 to 5 slots at d = 32, 3 the fastest)
  static constexpr int REQ = TILEB / 1024;           // 1 KB requests per tile
  static constexpr int RPW = REQ / kWinWaves;        // requests per wave per tensor
  static constexpr int REQ_PER_WAVE = 3 * RPW;       // per item
  static constexpr int NKS = D / 16;                 // MFMA steps over d
  static constexpr int DVB = D / 32;                 // 32-wide blocks of d
  static constexpr int TBLB = 1024;                  // table, (2M - 1)^2 <= 225 floats
  static constexpr int LDS = S * SLOTB + TBLB + 256;  // + 64 key lengths
  static_assert(REQ % kWinWaves == 0, "requests must split over the waves");
};

// Lane part of request I of a 64-row tile (1 KB: lane l fills row
// r = I * RPI + l / CPR, chunk l % CPR, swizzled by the row, from global row
// min(r, row_max)): its byte offset from the tile's first global row.  The
// host admits only strides for which every offset fits 31 bits.
template <int ROWB>
__device__ __forceinline__ uint32_t win_lane_offset(int I, int64_t stride, int row_max, int lane) {
  constexpr int CPR = ROWB / 16, RPI = 1024 / ROWB;
  const int r = I * RPI + lane / CPR;
  const int cc = (lane % CPR) ^ chunk_swizzle<CPR>(r);
  return (uint32_t)((int64_t)min(r, row_max) * stride * 2 + cc * 16);
}

// wait until this wave's requests of every item after the current one (k of
// them, k < S) may still be in flight, i.e. the current item's have landed
template <int R, int K>
__device__ __forceinline__ void wait_items_after(int k) {
  static_assert(K * R <= 63, "vmcnt holds at most 63");
  if constexpr (K == 0) {
    wait_vm<0>();
  } else {
    if (k >= K) wait_vm<K * R>();
    else wait_items_after<R, K - 1>(k);
  }
}

template <int D>
__global__ __launch_bounds__(kWinThreads) __attribute__((amdgpu_waves_per_eu(2)))
void window_grid_kernel(const FwdParams p, int items_per_wg) {
  using G = WinGeo<D>;
  constexpr int NKS = G::NKS, DVB = G::DVB, ROWB = G::ROWB, S = G::S;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char RELATTN_LDS* smem_lds = (unsigned char RELATTN_LDS*)smem;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem_lds;
  const float* TBL = reinterpret_cast<const float*>(smem + S * G::SLOTB);
  const int32_t* KL = reinterpret_cast<const int32_t*>(smem + S * G::SLOTB + G::TBLB);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hh = lane >> 5;
  const int n = p.n, M = p.grid_m;
  const int total = p.B * p.H;
  // this workgroup's run of items: item = h * B + b (a run stays within a head
  // unless it crosses a head boundary)
  const int first = blockIdx.x * items_per_wg;
  const int last = min(first + items_per_wg, total);
  if (first >= last) return;
  const float sl2 = p.scale_log2;
  const int qrow = wave * 32 + ql;

  auto item_bh = [&](int it, int& b, int& h) __attribute__((always_inline)) {
    h = it / p.B;
    b = it - h * p.B;
  };
  // this wave's requests of every item: tensor t (Q, K, V), request
  // I = wave + 2u of its tile, at lane offsets that hold for every item
  uint32_t voff[3][G::RPW];
#pragma unroll
  for (int u = 0; u < G::RPW; ++u) {
    const int I = wave + kWinWaves * u;
    voff[0][u] = win_lane_offset<ROWB>(I, p.q_sn, n - 1, lane);
    voff[1][u] = win_lane_offset<ROWB>(I, p.k_sn, n - 1, lane);
    voff[2][u] = win_lane_offset<ROWB>(I, p.v_sn, n - 1, lane);
  }
  // requests of item `it` into slot s
  auto request = [&](int it, int s) __attribute__((always_inline)) {
    int b, h;
    item_bh(it, b, h);
    const unsigned char* base[3] = {
        reinterpret_cast<const unsigned char*>(p.q) + 2 * (b * p.q_sb + h * p.q_sh),
        reinterpret_cast<const unsigned char*>(p.k) + 2 * (b * p.k_sb + h * p.k_sh),
        reinterpret_cast<const unsigned char*>(p.v) + 2 * (b * p.v_sb + h * p.v_sh)};
    unsigned char RELATTN_LDS* slot = smem_lds + s * G::SLOTB + wave * 1024;
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int u = 0; u < G::RPW; ++u)
        __builtin_amdgcn_global_load_lds(
            (const RELATTN_GLOBAL void*)(base[t] + voff[t][u]),
            (RELATTN_LDS void*)(slot + t * G::TILEB + kWinWaves * u * 1024), 16, 0, 0);
    compiler_fence();
  };
  // The head's bias table and the key lengths of up to 64 items of the run
  // reach LDS by DMA like the items (4 bytes a lane, wave 0 the table, wave 1
  // the lengths), so that every vector load is covered by the explicit waits:
  // the compiler cannot count loads in order past LDS-DMA and waits for all of
  // them before using any loaded register.
  const int nb = (2 * M - 1) * (2 * M - 1);
  const bool has_kl = p.key_lens != nullptr;
  auto table_request = [&](int h) __attribute__((always_inline)) {
    if (wave == 0) {
      const float* tb = p.t5_bias + (int64_t)h * p.tb_sh;
      for (int I = 0; I * 64 < nb; ++I)
        __builtin_amdgcn_global_load_lds(
            (const RELATTN_GLOBAL void*)(tb + (int64_t)min(I * 64 + lane, nb - 1) * p.tb_sb),
            (RELATTN_LDS void*)(smem_lds + S * G::SLOTB + I * 256), 4, 0, 0);
    }
    compiler_fence();
  };
  int kl_base = first;  // item of KL[0]
  auto lens_request = [&](int base) __attribute__((always_inline)) {
    if (has_kl && wave == kWinWaves - 1) {
      const int itl = min(base + lane, last - 1);
      __builtin_amdgcn_global_load_lds((const RELATTN_GLOBAL void*)(p.key_lens + itl % p.B),
                                       (RELATTN_LDS void*)(smem_lds + S * G::SLOTB + G::TBLB),
                                       4, 0, 0);
    }
    compiler_fence();
  };
  // this lane's bias for its query row and keys from the staged table:
  // register (kb, 8g + e) holds key 32kb + 16g + 8hh + e, log2 units, -inf
  // past n (rows and keys past n read a clamped entry, then take -inf; every
  // read is unconditional and pinned before the select, which the compiler
  // would otherwise turn into a branch around each read)
  float bv[2][16];
  auto bias_build = [&]() __attribute__((always_inline)) {
    const int qi = min(qrow, n - 1), yi = qi / M, xi = qi - yi * M;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = 32 * kb + 16 * (r >> 3) + 8 * hh + (r & 7);
        const int jj = min(j, n - 1), yj = jj / M, xj = jj - yj * M;
        const bool ok = qrow < n && j < n;
        float t = TBL[(yj - yi + M - 1) * (2 * M - 1) + (xj - xi + M - 1)];
        asm volatile("" : "+v"(t));
        bv[kb][r] = ok ? kLog2e * t : kNegInf;
      }
  };

  // ---- prologue: the head's table and the run's key lengths, the first S - 1
  // items' requests (a short run re-requests its last item into unused slots,
  // which keeps the wait counts below exact), then the head's bias once the
  // table has landed
  int hb, bb;
  item_bh(first, bb, hb);
  table_request(hb);
  lens_request(first);
#pragma unroll
  for (int u = 0; u < S - 1; ++u) request(min(first + u, last - 1), u);
  wait_vm<(S - 1) * G::REQ_PER_WAVE>();
  block_sync();
  bias_build();
  int h_cur = hb;

  // lane's K fragment offsets (row k_row_of_mfma_row(ql) of a 32-key block,
  // chunk 2ks + hh) and V^T transpose-read bases within a tile
  uint32_t kfo[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    kfo[ks] = (uint32_t)tile_offset<ROWB>(k_row_of_mfma_row<true>(ql), (2 * ks + hh) * 16);
  uint32_t trb_lo[DVB], trb_hi[DVB];
#pragma unroll
  for (int mb = 0; mb < DVB; ++mb) frag_col_base<ROWB, D>(32 * mb, lane, trb_lo[mb], trb_hi[mb]);

  int s = 0;  // slot of item `it`
  for (int it = first; it < last; ++it) {
    int b, h;
    item_bh(it, b, h);
    block_sync();  // every wave is done with the previous item and the table
    // a new head's table, or the next 64 items' key lengths (each waits for
    // the items in flight)
    const bool new_head = h != h_cur, new_lens = has_kl && it - kl_base >= 64;
    if (new_head || new_lens) {
      if (new_head) table_request(h);
      if (new_lens) {
        kl_base = it;
        lens_request(it);
      }
      wait_vm<0>();
      block_sync();
      if (new_head) bias_build();
      h_cur = h;
    }
    // item it + S - 1 into the slot the previous item freed
    const int ahead = it + S - 1;
    if (ahead < last) request(ahead, s == 0 ? S - 1 : s - 1);
    wait_items_after<G::REQ_PER_WAVE, S - 1>(min(last - 1, ahead) - it);
    block_sync();  // ... and for both waves

    const uint32_t slot = smem_addr + (uint32_t)(s * G::SLOTB);
    const unsigned char* Qt = smem + s * G::SLOTB;
    s = s == S - 1 ? 0 : s + 1;
    // key range of this window
    int kv_len = n;
    if (has_kl) kv_len = __builtin_amdgcn_readfirstlane(min(max(KL[it - kl_base], 0), n));

    // S^T = K Q^T for keys 0-31 (kb = 0) and 32-63 (kb = 1)
    bf16x8 qop[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qop[ks] = frag_row<ROWB>(Qt, qrow, 2 * ks + hh);
    f32x16 sacc[2];
    {
      bf16x8 a[2][NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint32_t ad = slot + (uint32_t)G::TILEB + kfo[ks];
        asm volatile("ds_read_b128 %0, %1" : "=v"(a[0][ks]) : "v"(ad));
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(a[1][ks]) : "v"(ad), "n"(32 * ROWB));
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+v"(a[0][ks]), "+v"(a[1][ks]));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) sacc[kb] = mfma(a[kb][ks], qop[ks], sacc[kb]);
      }
    }
    // logits: register (kb, 8g + e) holds key 32kb + 16g + 8hh + e; keys past
    // the window's length masked only on the path that needs it (the compiler
    // would otherwise turn the uniform test into a select per logit)
    float mx = kNegInf;
    auto logits = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = fmaf(sacc[kb][r], sl2, bv[kb][r]);
          if constexpr (decltype(masked)::value)
            x = (32 * kb + 16 * (r >> 3) + 8 * hh + (r & 7) < kv_len) ? x : kNegInf;
          sacc[kb][r] = x;
          mx = __builtin_elementwise_maximum(mx, x);
        }
    };
    if (kv_len < n) logits(std::true_type{});
    else logits(std::false_type{});
    {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                      false, false);
      mx = __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    const float m_use = (mx == kNegInf) ? 0.f : mx;
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[kb][t2][e] = (__bf16)fast_exp2(sacc[kb][8 * t2 + e] - m_use);
    // the normaliser sums the rounded weights the product uses, two at a time
    float psum;
    {
      bf16x2 one;
      one[0] = (__bf16)1.f;
      one[1] = (__bf16)1.f;
      float acc2[2] = {0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
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
    const float l = halves_sum(psum);
    const float inv_l = l > 0.f ? 1.f / l : 0.f;

    // O^T = V^T P^T
    f32x16 oacc[DVB];
#pragma unroll
    for (int mb = 0; mb < DVB; ++mb) oacc[mb] = f32x16{};
    const uint32_t vt = slot + (uint32_t)(2 * G::TILEB);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x4 vlo[2 * DVB], vhi[2 * DVB];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb)
          frag_col_issue_blk<ROWB>(2 * kb + t2, vt + trb_lo[mb], vt + trb_hi[mb],
                                   vlo[t2 * DVB + mb], vhi[t2 * DVB + mb]);
      frag_col_wait(vlo, vhi);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int mb = 0; mb < DVB; ++mb)
          oacc[mb] = mfma(frag_join(vlo[t2 * DVB + mb], vhi[t2 * DVB + mb]), pb[kb][t2],
                          oacc[mb]);
    }
    if (qrow < n) {
      __bf16* orow = reinterpret_cast<__bf16*>(p.o) + b * p.o_sb + h * p.o_sh +
                     (int64_t)qrow * p.o_sn;
#pragma unroll
      for (int mb = 0; mb < DVB; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[mb][4 * g + e] * inv_l);
          *reinterpret_cast<bf16x4*>(orow + 32 * mb + 8 * g + 4 * hh) = o4;
        }
      // row statistic for the backward pass, natural log
      if (p.lse && hh == 0)
        p.lse[b * p.lse_sb + h * p.lse_sh + qrow] = l > 0.f ? (m_use + log2f(l)) * kLn2 : kNegInf;
    }
  }
}

template <int D>
int window_launch_t(const FwdParams& p, void* stream) {
  using G = WinGeo<D>;
  auto kern = window_grid_kernel<D>;
  static std::atomic<int> lds_set[64];
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), G::LDS, lds_set);
  if (e != hipSuccess) return (int)e;
  // enough workgroups to fill every CU to its LDS-bound occupancy, each with a
  // contiguous run of items
  const long long items = (long long)p.B * p.H;
  const long long per_cu = 160 * 1024 / G::LDS;
  const long long target = 256 * (per_cu < 1 ? 1 : per_cu);
  const long long run = (items + target - 1) / target;
  const long long grid = (items + run - 1) / run;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kWinThreads), G::LDS,
                     reinterpret_cast<hipStream_t>(stream), p, (int)run);
  return (int)hipGetLastError();
}

}  // namespace

bool window_grid_ok(bool bf16, int d, int n, int grid_m, int64_t max_row_stride) {
  // lane offsets within a tile are 32-bit (rows below 64 of 2-byte elements)
  const bool offsets_fit = max_row_stride >= 0 &&
                           max_row_stride < ((int64_t)1 << 31) / (2 * kWinRows) - 64;
  return bf16 && (d == 32 || d == 64) && n <= kWinRows && grid_m >= 1 && grid_m <= 8 &&
         offsets_fit;
}

int launch_window_grid(int d, const FwdParams& p, void* stream) {
  if (d == 32) return window_launch_t<32>(p, stream);
  if (d == 64) return window_launch_t<64>(p, stream);
  return (int)hipErrorInvalidValue;
}

}  // namespace relattn
