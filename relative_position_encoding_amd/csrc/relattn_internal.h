// Internal interface between the C-ABI host code (relattn_api.cpp) and the
// gfx950 kernels (relattn_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <stdint.h>

namespace relattn {

constexpr int kMaxT5Thresholds = 64;

// Bucket function of the T5 section, in the form the kernels evaluate it.
// thr[t] is the smallest distance a whose logarithmic bucket index
// floor(nlog * ln(a / exact) / ln(D_max / exact)) is at least t + 1; the host
// derives it with exact integer arithmetic.
struct T5Buckets {
  int32_t nb;       // number of buckets (rows of the bias table)
  int32_t half;     // buckets per sign (bidirectional) or all buckets
  int32_t exact;    // B_exact = half / 2
  int32_t nlog;     // half - exact logarithmic buckets
  int32_t bidir;
  int32_t thr[kMaxT5Thresholds];
};

// Everything a forward launch needs.  Strides count elements.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const void* wk;          // [Ht, 2c+1, d] or null
  const void* wv;          // [Ht, 2c+1, d] or null
  const float* t5_bias;    // [NB, H] or null
  const int32_t* key_lens; // [B] or null

  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t wk_sh, wk_sr;    // head stride 0 = shared table
  int64_t wv_sh, wv_sr;
  int64_t tb_sb, tb_sh;    // T5 bias strides: bucket, head

  int32_t B, H, n;
  int32_t clip;            // c of clip(j - i, c)
  int32_t r_lo, nr;        // label rows reachable: [r_lo, r_lo + nr)
  int32_t causal;
  float scale_log2;        // logit scale times log2(e)
  int32_t t5_dist;         // offsets are clamped to [-t5_dist, t5_dist]
  int32_t n_qtiles;        // query tiles per (b, h)
  int32_t nstage;          // K/V tiles in the LDS ring (2 or 3)
  int32_t wv_mode;         // WvMode: where the w^V tile is staged
  int32_t dma32;           // K/V tile rows fit 32-bit byte offsets (fast stage loads)
  // Divisions of workgroup ids (< 2^31) by H, by the query tiles per head and by
  // the heads per XCD, as x / d == (umulhi(x, m) + x) >> s (host-computed; the
  // lean kernel's tile mapping uses them instead of a division sequence).
  uint32_t dv_h_m, dv_qt_m, dv_hpx_m;
  int32_t dv_h_s, dv_qt_s, dv_hpx_s;
  // The scalar-bias arm takes either T5 buckets (ob = 0: t5_bias is [NB, H])
  // or a table by clipped offset (ob = 1: t5_bias points at the head's row of
  // a [Hb, 2W + 1] table; t5.nb = 2 * t5_dist + 1 entries starting at ob_lo
  // = W - t5_dist are loaded).
  int32_t ob;
  int32_t ob_lo;
  // Optional row statistics: lse[b * lse_sb + h * lse_sh + i] receives the
  // natural-log log-sum-exp of row i's visible logits (-inf for none).
  float* lse;
  int64_t lse_sb, lse_sh;
  // Transformer-XL (xl = 1): the key table is the position table R read by
  // i - j, and the query is shifted by the head's global bias u for the content
  // logit and v for the relative logit.  Shaw mode with the key table only
  // (d = 128): wk starts at R's last row with a negative row stride; XL mode
  // (d <= 64): wk points at R's row of distance 0.
  const void* xl_u;
  const void* xl_v;
  int64_t xl_u_sh, xl_v_sh;  // head strides (0 = one vector for all heads)
  int32_t xl;
  // 2-D window bias (grid mode, grid_m = M > 0, ob = 1): tokens in
  // raster order on an M x M grid; t5_bias points at the head's row of a
  // [Hb, (2M-1)^2] table and t5.nb = (2M-1)^2 entries are loaded.
  int32_t grid_m;
  float grid_inv;  // 1 / M
  // Edge labels (label and graph modes): lab[b * lab_sb + i * lab_sn + j] is
  // the label of the edge from query i to key j; rows are read in whole
  // 16-byte chunks (lab_sn a multiple of 16, at least n rounded up to 16).
  // Label mode: t5_bias points at the head's row of a [Hb, NL] table and
  // t5.nb = NL.  Graph mode: wk / wv are [Ht, NL, d] tables, r_lo = 0, nr = NL.
  const uint8_t* lab;
  int64_t lab_sb, lab_sn;
  T5Buckets t5;
};

// kRelT5: scalar bias by T5 bucket or clipped offset; kRelLabel: scalar bias
// by a per-pair label read from memory; kRelGrid: scalar bias by the 2-D
// offset of raster tokens on an M x M window; kRelXL: Transformer-XL with the
// relative logits formed per key tile (wk points at the position table's row of
// distance 0, rows by distance i - j clamped to +-clip).
// kRelGraph: the Shaw key/value tables indexed by a per-pair label (lab as for
// kRelLabel; r_lo = 0, nr = NL table rows).
enum RelMode { kRelNone = 0, kRelShaw = 1, kRelT5 = 2, kRelLabel = 3, kRelGrid = 4,
               kRelXL = 5, kRelGraph = 6 };

// Where the w^V rows wait for the epilogue: their own LDS region (loaded in
// the prologue), the first K/V ring stage the loop frees, or the free ring
// after the loop in chunks.
enum WvMode { kWvResident = 0, kWvRing = 1, kWvChunked = 2 };

// Kernel configuration picked by the host for one call.
struct LaunchCfg {
  int waves;   // 32 query rows per wave
  int kblock;  // keys per tile
  int nstage;  // K/V tiles in the LDS ring
  int wv_mode;  // WvMode (general kernel)
  int lean = 0;  // 1: the lean bf16 kernel (relattn_fwd_bf16.hip); 3: the small-window kernel
};

// Dynamic LDS bytes of one workgroup (same layout function as the kernel);
// SIZE_MAX when the configuration cannot hold the tables.
size_t lds_bytes(bool bf16, int d, const LaunchCfg& cfg, RelMode mode, bool has_wk,
                 bool has_wv, int nr, int t5_dist, int t5_nb);

// The lean bf16 kernel (relattn_fwd_bf16.hip): bf16, d = 64, 64-key tiles, 4 or
// 8 waves, the Shaw tables, the T5 / clipped-offset
// scalar bias or no relative term.  Its tables and relative rows stay resident
// in LDS; the ring prefetches every tile of a workgroup when nstage covers them.
bool lean_mode_ok(bool bf16, int d, RelMode mode);
size_t lean_lds_bytes(int d, const LaunchCfg& cfg, RelMode mode, bool has_wk, bool has_wv,
                      int nr, int t5_dist, int t5_nb);
int launch_fwd_lean(int d, const LaunchCfg& cfg, RelMode mode, bool has_wk, bool has_wv,
                    const FwdParams& p, void* stream);

// The persistent small-window kernel of the 2-D window bias
// (relattn_window.hip): bf16, d = 32 or 64, windows of at most 64 tokens
// (M <= 8), row strides below 2^24 elements; each workgroup walks a run of
// (window, head) items through a ring of LDS slots, the next items' rows
// requested during the current one.
bool window_grid_ok(bool bf16, int d, int n, int grid_m, int64_t max_row_stride);
int launch_window_grid(int d, const FwdParams& p, void* stream);

// Launchers (relattn_kernels.hip).  Return a hipError_t value.
int launch_fwd(bool bf16, int d, const LaunchCfg& cfg, RelMode mode, bool has_wk,
               bool has_wv, const FwdParams& p, void* stream);
int launch_debug_indices(int n, int clip, const T5Buckets* t5, int32_t* out,
                         void* stream);

// ---- backward (relattn_backward.hip) --------------------------------------

// Everything the three backward launches need.  Strides count elements.
// Workspace sections (fp32):
//   ws_stat [B*H][2][n_pad] + 64 : per query, lse in log2 units and D = dz.z
//   ws_pk   [B*H][n_qtiles][nr][d], ws_pv the same : per query-tile partial
//                                  table gradients (ws_pk already scaled)
//   ws_pb   [B*H][n_qtiles][nb]  : per query-tile partial bias gradients
//   ws_pu   [B*H][n_qtiles][2][d]: Transformer-XL, per query tile, its rows'
//                                  sums of the content and the relative part
//                                  of dq (unscaled)
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;            // forward output z
  const void* dout;         // dz
  const float* lse;         // [B, H, n] natural log
  const void* wk;
  const void* wv;
  const float* t5_bias;
  const int32_t* key_lens;
  void* dq;
  void* dk;
  void* dv;
  float* dwk;               // [Htk, 2c+1, d] or null
  float* dwv;
  float* db;                // T5: [NB, H]; offset bias: [Hb, 2W+1]; 2-D window: [Hb, (2M-1)^2]; or null
  float* ws_stat;
  float* ws_pk;
  float* ws_pv;
  float* ws_pb;

  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t do_sb, do_sh, do_sn;
  int64_t dq_sb, dq_sh, dq_sn;
  int64_t dk_sb, dk_sh, dk_sn;
  int64_t dv_sb, dv_sh, dv_sn;
  int64_t lse_sb, lse_sh;
  int64_t wk_sh, wk_sr;
  int64_t wv_sh, wv_sr;
  int64_t tb_sb, tb_sh;
  int64_t dwk_sh, dwk_sr;   // output table gradients
  int64_t dwv_sh, dwv_sr;
  int64_t db_s0, db_s1;     // bias gradient strides (dims 0 and 1 of its shape)

  int32_t B, H, n, d;
  int32_t n_pad;            // n rounded up to 64
  int32_t clip;
  int32_t r_lo, nr;         // reachable labels [r_lo, r_lo + nr)
  int32_t htk, htv;         // table heads (H or 1)
  int32_t hb;               // bias gradient heads (offset bias: H or 1)
  int32_t causal;
  float scale;              // logit scale s
  float scale_log2;         // s * log2(e)
  int32_t t5_dist;
  int32_t ob, ob_lo;        // scalar bias from a [hb, ob_n] table (ob = 1)
  int32_t ob_n;             // its entries per row: 2W + 1 by clipped offset, (2M-1)^2 by
                            // 2-D offset, NL by edge label
  int32_t n_qtiles;         // query tiles per (b, h) of the dq kernel
  int32_t n_ktiles;         // key tiles per (b, h) of the dk/dv kernel
  T5Buckets t5;
  // (the modes below read fields of their own, kept after the common ones)
  int32_t grid_m;           // 2-D window: side M (n = M * M); its table has (2M-1)^2 entries
  float grid_inv;           // 1 / M
  // edge labels: lab[b * lab_sb + i * lab_sn + j] labels the pair (query i,
  // key j); rows are readable in whole 16-byte chunks up to n rounded up to 16
  const uint8_t* lab;
  int64_t lab_sb, lab_sn;
  // Transformer-XL (mode kRelXL, the Shaw key-table path): wk is R read by
  // i - j (its last row, negative row stride); the content logit takes q + u
  // and the relative logit q + v.  du, dvb: [hu, d] and [hv, d] fp32 outputs
  // (NULL to skip).
  const void* xl_u;
  const void* xl_v;
  int64_t xl_u_sh, xl_v_sh;
  float* du;
  float* dvb;
  int64_t du_sh, dvb_sh;
  int32_t hu, hv;
  float* ws_pu;
  // tables by edge label: rows per head of each table (0: 2 clip + 1)
  int32_t nlab;
};

struct BwdCfg {
  int qwaves, qkblock;  // dq kernel: waves (32 query rows each), keys per tile
  int kwaves, kqblock;  // dk/dv kernel: waves (32 key rows each), queries per tile
};

// Workgroup shapes the backward kernels are built with: the wide ones, or the
// narrow ones (half the query rows of the dq kernel, or half the queries per
// tile of the dk/dv kernel) that fit larger label windows on chip; for the
// widest windows of the key-table modes in bf16 at d <= 64, a tiny dq shape
// (one wave, 32-key tiles).
BwdCfg bwd_cfg(bool bf16, int d, bool narrow_q, bool narrow_kv, bool tiny_q = false);
size_t bwd_lds_q(bool bf16, int d, const BwdCfg& cfg, RelMode mode, bool has_wk, bool has_wv,
                 int nr, int t5_dist, int nb, bool want_db);
size_t bwd_lds_kv(bool bf16, int d, const BwdCfg& cfg, RelMode mode, bool has_wk, bool has_wv,
                  int nr, int t5_dist, int nb);
int launch_bwd(bool bf16, int d, const BwdCfg& cfg, RelMode mode, bool has_wk, bool has_wv,
               const BwdParams& p, void* stream);

// ---- incremental decoding (relattn_decode.hip) ----------------------------

// Keys of the cache one decode workgroup streams per step of its loop: 32 KB
// of K rows, i.e. eight 16-byte loads of K (and of V) per lane of a
// 256-thread workgroup.
constexpr int dec_chunk(int elem_bytes, int d) { return 32768 / (elem_bytes * d); }
// Workgroups a decode launch aims for (four per compute unit), and the most
// single-key labels a workgroup that owns a whole row keeps in LDS.
constexpr int kDecTargetWgs = 1024;
constexpr int kDirectBand = 1024;

// Everything a decode launch needs.  Query t of batch b sits at position
// cache_lens[b] - Tq + t of its sequence.  Strides count elements.  The
// workspace holds, per query row (b, h, t) and chunk, the partial max and sum
// (ws_ml, 2 floats) and the partial output (ws_o, d floats), and per row the
// raw logits of the keys whose label holds them alone (ws_band, nband floats).
struct DecParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const void* wk;
  const void* wv;
  const float* t5_bias;
  const int32_t* cache_lens;  // [B] or null (every row of the cache is valid)
  float* ws_ml;
  float* ws_o;
  float* ws_band;

  int64_t q_sb, q_sh, q_st;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_st;
  int64_t wk_sh, wk_sr;
  int64_t wv_sh, wv_sr;
  int64_t tb_sb, tb_sh;

  int32_t B, H, Tq, L;  // L = rows of the cache
  int32_t clip;
  int32_t nband;        // min(clip, L) with a value table, else 0
  int32_t nch;          // chunks per query row: ceil(L / dec_chunk)
  int32_t cps;          // chunks per split: one workgroup streams a split
  int32_t nsp;          // splits per query row: ceil(nch / cps)
  int32_t direct;       // nsp == 1 and the row's single-key labels fit in LDS:
                        // one workgroup per row writes the output itself
  float scale_log2;
  // scalar-bias mode with ob = 1: t5_bias points at a [Hb, 2W + 1] table by
  // clipped offset (entry clip(delta, W) + W, W = ob_w) instead of T5 buckets
  int32_t ob;
  int32_t ob_w;
  // Transformer-XL (XL mode): wk is the position table R [Hr, 2 clip + 1, d]
  // (row clip + (i - j)); u and v shift the query for the content and the
  // position term (head strides 0 = shared)
  const void* xl_u;
  const void* xl_v;
  int64_t xl_u_sh, xl_v_sh;
  T5Buckets t5;
};

// Launch the partial and combine kernels.  Returns a hipError_t value.
int launch_decode(bool bf16, int d, RelMode mode, bool has_wk, bool has_wv,
                  const DecParams& p, void* stream);

}  // namespace relattn
