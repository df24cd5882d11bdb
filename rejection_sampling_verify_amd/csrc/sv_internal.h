// sv_internal.h — argument blocks and workspace records shared by the host
// launchers and the kernels of the verify library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kMaxSets = 8;           // ticket queues (one per XCD of an MI355X)
constexpr int kTicketStride = 1024;   // words between ticket counters (4 KiB)
constexpr int kMaxVecsPerThread = 8;  // 16-byte vectors per thread per row chunk
constexpr int kMaxGamma = 16;
constexpr int kMaxTreeNodes = 1024;

// Pass-2 work of a decided sequence.
enum P2Mode : uint32_t {
  P2_NONE = 0,            // output complete after the decision
  P2_RESIDUAL = 1,        // Gumbel-max over ln (p - q)_+ of row `row`
  P2_RESIDUAL_ONEHOT = 2, // Gumbel-max over l/T of row `row`, excluding `x`
  P2_BONUS = 3,           // Gumbel-max over l/T of row gamma
  P2_GREEDY_BONUS = 4     // argmax of row gamma
};

// Per-sequence record in the workspace (64 bytes). All fields are zero
// between calls.
struct SeqState {
  uint32_t p1_arrive;  // pass-1 items finished
  uint32_t p2_arrive;  // pass-2 items finished
  uint32_t flag;       // 1 once the decision and the fields below are published
  uint32_t mode;       // P2Mode
  int32_t row;         // row position of the pass-2 draw
  int32_t x;           // drafted id at `row` (excluded by the one-hot residual)
  float logz2_t;       // log2-domain normalizer of target row `row`
  float logz2_d;       // same for the draft row
  uint32_t error;      // nonzero: a bounded wait gave up
  int32_t n;           // accepted drafts
  uint32_t pad[6];
};

struct P1Partial {  // sampled rows: (Mt, st, Md, sd); greedy rows: (value, index bits, 0, 0)
  float a, b, c, d;
};

struct Gathered {  // raw logits of the drafted id in its target / draft row
  float lt, ld;
};

struct P2Partial {
  float score;
  int32_t idx;
  float beta;
  int32_t any;  // the chunk held at least one candidate
};

struct TreePartial {
  float v;
  int32_t i;
};

struct ChainArgs {
  const uint8_t* target;
  int64_t t_stride;  // bytes between rows
  const uint8_t* draft;  // NULL: one-hot draft
  int64_t d_stride;
  const int32_t* ids;          // [B, gamma]
  const float* temperature;    // [B] or NULL: every sequence greedy
  int32_t B, gamma, V;
  int32_t chunk;    // elements per chunk
  int32_t nchunks;  // chunks per row
  int32_t kv;       // 16-byte vectors per thread per chunk (<= kMaxVecsPerThread)
  uint32_t key0, key1;
  uint32_t ctr_accept, ctr_noise;  // counter word 3 of the two Philox streams
  int32_t* out_tokens;
  int32_t* out_n;
  float* d_accept;
  float* d_logzt;
  float* d_logzd;
  float* d_beta;
  uint32_t* tickets;  // [kMaxSets * kTicketStride]
  uint32_t* done;     // [0]: workgroups finished; [1]: a bounded wait gave up
  SeqState* seq;      // [B]
  P1Partial* p1;      // [B, gamma, nchunks]
  Gathered* gath;     // [B, gamma]
  P2Partial* p2;      // [B, nchunks]
  int32_t nsets;
  int32_t lag;        // pass-2 items of local sequence k follow pass-1 items of k + lag
  int32_t fused;      // pass-2 items share the ticket queues with pass 1
  uint32_t spin_limit;
};

struct TreeArgs {
  const uint8_t* target;
  int64_t t_stride;
  const int32_t* parents;
  const int32_t* depth;
  const int32_t* tokens;  // [B, N]
  int32_t B, N, V, max_depth;
  int32_t chunk, nchunks, kv;
  int32_t* out_path;
  int32_t* out_path_len;
  int32_t* out_bonus;
  uint32_t* arrive;       // [B]
  TreePartial* part;      // [B, N, nchunks]
};

// Workspace carve-up; every offset is a multiple of 256 bytes.
struct WsLayout {
  size_t tickets, done, seq, p1, gath, p2, tree_arrive, tree_part, total;
};

WsLayout ws_layout(int32_t B, int32_t rows, int32_t nchunks);
int32_t max_chunks(int32_t V);

// Launchers (host). Return hipSuccess or the first HIP error.
hipError_t launch_chain(const ChainArgs& a, bool bf16, bool vec, int grid, hipStream_t stream);
hipError_t launch_chain_p2(const ChainArgs& a, bool bf16, bool vec, hipStream_t stream);
hipError_t launch_tree(const TreeArgs& a, bool bf16, bool vec, hipStream_t stream);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
int chain_occupancy(bool bf16, bool vec);

}  // namespace sv
