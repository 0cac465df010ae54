// Launchers of the gfx950 MoE kernels (internal; used by api.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Routing description handed to the selection code.
struct RouteParams {
  int T, H, E, k;
  int G, gsz, topk_group;
  int scoring;   // 0 softmax, 1 sigmoid, 2 sqrt(softplus)
  int renorm;
  float scale;
  int capacity;  // <= 0: unlimited
  int n_allowed; // experts a token may pick from after the group limit
};

struct RouterArgs {
  RouteParams p;
  const void* x;            // [T,H] (fused fp32 router only)
  const void* w_router;     // [E,H] (fused fp32 router only)
  const float* part;        // selection kernel: [nsplit,T,E] partial logits without bias
  int nsplit;               //   (summed in order, then logit_bias added)
  const float* logit_bias;  // [E] or null
  const float* sel_bias;    // [E] or null
  const float* logits_in;   // [T,E] or null: route these logits
  float* logits_out;        // [T,E] or null
  int32_t* topk_idx;        // [T,k] (unused in capacity mode)
  float* topk_w;            // [T,k]
  int32_t* counts;          // [E] atomically incremented, or null
  int32_t* cand;            // capacity mode: [T,n_allowed] experts in rank order
  int hash;                 // 1: hash routing through token_ids and tid2eid
  const int32_t* token_ids; //   [T] token ids
  const int32_t* tid2eid;   //   [vocab,k] expert table (unread when vocab == 0)
  int64_t vocab;
};

// Router GEMM (bf16): logits of 64-token tiles over K slices of sps steps of
// 64; out is [T,E] when S == 1, else [S,T,E] partial sums.
struct RouterGemmArgs {
  int T, H, E, S, sps;
  const void* x;            // [T,H]
  const void* w;            // [E,H]
  float* out;
};

struct CapacityArgs {
  RouteParams p;
  const float* logits;      // [T,E]
  const int32_t* cand;      // [T,n_allowed]
  int32_t* topk_idx;        // [T,k]
  float* topk_w;            // [T,k]
  int32_t* counts;          // [E] or null
};

struct PermuteArgs {
  int T, E, k, S, nchunks;
  const int32_t* topk_idx;  // [T,k]
  int32_t* chunk_cnt;       // [nchunks,E]
  int32_t* chunk_base;      // [nchunks,E]
  int32_t* counts;          // [E]
  int32_t* offsets;         // [E+1]
  int32_t* row_token;       // [T*k + S*T]
  int32_t* slot_row;        // [T,k]
};

// Drop mode of the capacity limit: with the permutation of the unlimited
// top-k, assignment (t, j) to expert e has rank slot_row - offsets[e] among
// e's assignments in token order; ranks >= capacity are dropped.
struct DropArgs {
  int T, E, k, capacity;
  int32_t* topk_idx;        // [T,k] in/out: dropped slots become -1
  float* topk_w;            // [T,k] in/out: dropped slots get gate 0
  const int32_t* slot_row;  // [T,k] rows of the unlimited permutation
  const int32_t* offsets;   // [E+1]
  const int32_t* full_counts; // [E] assignments before the limit
  int32_t* counts;          // [E] out: min(full, capacity), or null
};

// Row segments of the experts (routed then shared) and the prefixes of their
// row-tile counts: full row tiles (more than half_rows rows) and short last
// row tiles (at most half_rows rows; half_rows = 0 makes every tile full).
struct ScheduleArgs {
  int T, E, S, k, BM, half_rows;
  const int32_t* offsets;   // [E+1]
  int32_t* seg_start;       // [E+S]
  int32_t* seg_len;         // [E+S]
  int32_t* f_prefix;        // [E+S+1] full row tiles before expert e
  int32_t* h_prefix;        // [E+S+1] short row tiles before expert e
  int32_t* pool;            // [2] item counters of the two GEMMs' shared pools, zeroed here
};

struct GemmArgs {
  int K, N;                 // reduction length, output columns of this GEMM
  int n_exp;                // E + S
  int n_tiles;              // column tiles per m-tile
  const void* a;            // gate/up: x [T,H]; down: h [rows,I]
  uint32_t a_bytes;         // gate/up: bytes of x (< 2^31: the gather addresses it through one buffer resource)
  const int32_t* row_token; // gate/up: token of every row
  const void* b0;           // gate/up: w_gate; down: w_down
  const void* b1;           // gate/up: w_up; down: unused
  void* c;                  // gate/up: h [rows,I]; down: y_rows [rows,H]
  const int32_t* seg_start;
  const int32_t* seg_len;
  const int32_t* f_prefix;
  const int32_t* h_prefix;
  // down, split output: routed experts' rows (experts < n_routed, rows <
  // routed_rows) to c16 in bf16, shared experts' rows to c (fp32) at row
  // minus routed_rows; c16 == null: every row to c (fp32)
  void* c16;
  int n_routed, routed_rows;
  // FP8 experts: a, b0, b1 and (gate/up) c hold E4M3 codes; UE8M0 scales of
  // A per row of the row space and 128-wide K block in the grouped layout
  // [ceil(K/512), n_rows, 4] (byte kb%4 of row r's dword in group kb/4: one
  // dword load brings four K steps, the rows of a tile are contiguous), of B
  // per 128 x 128 block with rows padded to a multiple of 4 bytes, of h like A's
  const uint8_t* sa;        // grouped [ceil(K/512), n_rows, 4]
  int n_rows;               // rows of the row space (T*k + S*T)
  const uint8_t* sb0;       // [n_exp, N/128, roundup(K/128, 4)] scales of b0, 4-byte aligned
  const uint8_t* sb1;       // the same for b1 (gate/up)
  uint8_t* sc;              // gate/up: grouped [ceil(N/512), n_rows, 4] scales of h
  // counter of the shared pool of items (the last sixteenth of every XCD's
  // range, taken by whichever XCD gets there first), zeroed before the
  // launch; null: every item stays with its XCD
  int32_t* pool;
  // down GEMM: 1 = its weights are copied with the non-temporal policy (each
  // weight tile read once, or mostly once); the gate/up GEMM chooses the
  // policy per item, from the item's expert, and ignores this field
  int stream_b;
  // bf16 down GEMM: 1 = three stages of input rows and two of weights
  int a3;
};

// Weight scales repacked with rows padded to 4 bytes (three matrices).
struct ScalePackArgs {
  struct Mat {
    int64_t rows;           // n_exp * (N/128)
    int nkb;                // K/128
    const uint8_t* src;     // [rows, nkb]
    uint8_t* dst;           // [rows, roundup(nkb, 4)]
  } m[3];
};

// Per-row copies of the tokens' x scales for the FP8 gate/up GEMM.
struct RowScaleArgs {
  int n_rows, nkb;
  const int32_t* row_token; // [n_rows], -1 = unused row
  const uint8_t* sx;        // [T, nkb] per token
  uint8_t* out;             // grouped [ceil(nkb/4), n_rows, 4]
};

// 1 x 128 tile quantisation of bf16 rows to E4M3 codes and UE8M0 scales.
struct QuantArgs {
  int64_t rows;
  int K;                    // multiple of 128
  const void* in;           // [rows, K] bf16
  uint8_t* codes;           // [rows, K]
  uint8_t* scales;          // [rows, sstride]
  int sstride;              // >= K/128
};

struct CombineArgs {
  int T, H, k, S;
  const void* y_routed;     // [T*k, H] routed expert rows, fp32 or bf16
  int routed_bf16;
  const float* y_shared;    // [S*T, H] shared expert rows (fp32)
  const int32_t* slot_row;  // [T,k]
  const float* topk_w;      // [T,k]
  void* out;                // [T,H]
};

// One balancing step (selection bias) and the load telemetry.
struct BalanceArgs {
  int E;
  const int32_t* counts;    // [E]
  float* bias;              // [E] selection bias, updated in place, or null
  float gamma;
  float* share;             // [E] or null
  float* stats;             // [4] or null: entropy (nats), max share, experts above / below the mean
};

// Kernel ids (for timing); names in kernel_names().
enum KernelId {
  K_FILL = 0,
  K_ROUTER,
  K_ROUTE_SELECT,
  K_CAPACITY,
  K_PERM_COUNT,
  K_PERM_SCAN,
  K_PERM_SCATTER,
  K_SCHEDULE,
  K_GATEUP,
  K_DOWN,
  K_COMBINE,
  K_BALANCE,
  K_QUANT,
  K_ROWSCALE,
  K_COUNT
};

const char* kernel_name(int id);

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
// Fused fp32 router (GEMM on fp32 MFMA + selection).
hipError_t launch_router(const RouterArgs& a, int dtype, hipStream_t s);
// K slices of the bf16 router GEMM for T tokens (>= 1) and E experts, and
// its launch.
int router_splits(int64_t T, int H, int E, int* sps);
hipError_t launch_router_gemm(const RouterGemmArgs& a, hipStream_t s);
// Selection from partial logits (a.part, a.nsplit) or from a.logits_in.
hipError_t launch_route_select(const RouterArgs& a, hipStream_t s);
hipError_t launch_capacity(const CapacityArgs& a, hipStream_t s);
hipError_t launch_perm_count(const PermuteArgs& a, hipStream_t s);
hipError_t launch_perm_scan(const PermuteArgs& a, hipStream_t s);
hipError_t launch_perm_scatter(const PermuteArgs& a, hipStream_t s);
hipError_t launch_drop(const DropArgs& a, hipStream_t s);
hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t s);
// Upper bound of the m-tiles of all experts (grid sizing without a host sync).
int64_t gemm_mtile_bound(int T, int E, int S, int k, int BM);
int gemm_bm(int dtype);
// Row count at or below which an expert's last row tile runs at half height.
int gemm_half_rows(int dtype);
hipError_t launch_gateup(const GemmArgs& a, int dtype, int64_t mtile_bound, hipStream_t s);
hipError_t launch_down(const GemmArgs& a, int dtype, int64_t mtile_bound, hipStream_t s);
// FP8 experts (gemm_fp8.hip): E4M3 operands with UE8M0 scales (GemmArgs sa,
// sb0, sb1, sc), and the 1 x 128 quantisation of bf16 rows.
hipError_t launch_gateup_fp8(const GemmArgs& a, int64_t mtile_bound, hipStream_t s);
hipError_t launch_down_fp8(const GemmArgs& a, int64_t mtile_bound, hipStream_t s);
hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t s);
hipError_t launch_row_scales(const RowScaleArgs& a, hipStream_t s);
hipError_t launch_pack_scales(const ScalePackArgs& a, hipStream_t s);
hipError_t launch_balance(const BalanceArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int dtype, int out_dtype, hipStream_t s);
// Attainable-rate probes (probe.hip): threads per block, FLOPs of one loop
// iteration of one block of the MFMA probe, and the launches.
int probe_threads();
double probe_mfma_flops_per_iter_block(int fp8);
// vary: four A and four B fragments in turn (1) or one fixed pair (0)
hipError_t launch_probe_mfma(int fp8, int vary, int blocks, int64_t iters, float* sink, hipStream_t s);
// mode 0: plain loads, 1: non-temporal loads, 2: global->LDS copies, 3: the
// same with the non-temporal policy
hipError_t launch_probe_read(int mode, int blocks, const void* buf, int64_t n16, float* sink, hipStream_t s);
