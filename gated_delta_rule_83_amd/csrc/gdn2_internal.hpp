// gdn2_internal.hpp -- launch interface between the C ABI layer and the
// kernels. Not installed; the public interface is include/gdn2.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn2 {

// Gate forms: per-channel fp32 gates; per-channel pre-activations in the
// input dtype; coupled b = w = beta (one fp32 per token and value head);
// scalar, also a = alpha (one fp32 per token and value head).
enum { kGateGeneral = 0, kGatePre = 1, kGateCoupled = 2, kGateScalar = 3 };

// Compute units of one MI355X (gfx950): one prefill workgroup each (its LDS
// working set admits one per unit), so this many make one round of a launch.
constexpr int kNumCU = 256;

struct DecodeArgs {
  int B, H_qk, H_v, d_k, d_v;
  bool bf16;
  const void *q, *k, *v;
  const void *a, *b, *w;  // layout and type by gate_form
  int gate_form;
  float *S;
  void *o;
};

struct PrefillArgs {
  int B, T, H_qk, H_v, d_k, d_v, chunk;
  bool bf16;
  int nct;  // 16-column state tiles per workgroup (one wave each): 1, 4 or 8
  const void *q, *k, *v;
  const float *a, *b, *w, *S0;
  void *o;
  float *S_T;
  void *workspace;  // split-sequence scratch (see PrefillPlan), may be null
  size_t workspace_bytes;
  // packed sequences of different lengths: B + 1 token offsets (device), or
  // null for B sequences of T tokens each
  const int32_t *cu_seqlens;
  // coupled gates: b and w both point to beta [.., T, H_v] (one scalar per
  // token and value head, b = w = beta * ones)
  bool coupled;
  // scalar decay (with coupled gates): a points to [.., T, H_v], one decay
  // per token and value head for all key channels
  bool scalar_decay;
  // per-channel gates given as pre-activations in the input dtype (a, b, w
  // point to them), activated in the kernel
  bool preact;
  // split into this many segments (0: the plan's own choice)
  int force_nseg;
  // the plan's own choice: at most this many workgroups in the split's first
  // pass (0: kNumCU, one round of the compute units)
  int split_wgs = 0;
  // states only (backward of long sequences): run the split's first two
  // passes and leave in seg_states[s] ([nseg][B][H_v][d_k][d_v]) the exact
  // state after segment s for s < nseg - 1; no outputs, no S_T; the
  // workspace holds the transition matrices (nseg * B * H_v * d_k^2 floats)
  float *seg_states;
  // largest workspace the split may use (0: no limit); a split whose
  // output-correction form needs more runs its segments a second time instead
  size_t ws_cap;
  // the state at every chunk boundary, in the input type (see
  // PrefillParams::cst); needs an unsplit plan (force_nseg = 1) and no
  // cu_seqlens
  void *chunk_states = nullptr;
  // chunk_states of B / cst_segs sequences, each given as cst_segs consecutive
  // segments of T tokens (PrefillParams::cst_segs); 1: whole sequences
  int cst_segs = 1;
};

// How a prefill call runs: the chunk length used (the largest supported one
// not above the requested one), and whether sequences are split into nseg
// segments of seg_len tokens processed in parallel (nseg = 1: unsplit), which
// needs ws_bytes of workspace.
struct PrefillPlan {
  int chunk, nseg, seg_len;
  size_t ws_bytes;
  // split form: true = outputs corrected from the identity columns' query
  // reads (one pass over the segments), false = segments run again from
  // their exact entering states
  bool correct;
};

// Thresholds on the decay per key channel above which the chunk-parallel form
// is used: of each half of the chunk where the Gram matrices are anchored at
// the chunk's middle (d_k = 128), of the whole chunk where they are anchored
// at its start. Below it the chunk is stepped token by token (exact for any
// decay). The operands carry at most the inverse of that decay, so every
// scale factor stays below e^60.
constexpr float kMinChunkDecay = 8.75651076e-27f;  // e^-60
constexpr float kMinHalfDecay = 8.75651076e-27f;   // e^-60
// per-chunk path of the prefill (flags of a chunk buffer): the chunk-start
// anchor (0), the middle-token anchor, or token by token
constexpr int kChunkSteps = 1;
constexpr int kChunkMid = 2;

// Backward pass (gradients of the recurrence); see gdn2_chunk_backward.
struct BackwardArgs {
  int B, T, H_qk, H_v, d_k, d_v;
  bool bf16;
  const void *q, *k, *v;
  const float *a, *b, *w, *S0;
  const void *dO;
  const float *dST;
  void *dq, *dk, *dv;
  float *da, *db, *dw, *dS0;
  void *workspace;  // 256-byte aligned
  size_t workspace_bytes;  // its size (what the launch may use)
  // packed sequences: B + 1 token offsets (device), or null for B sequences
  // of T tokens each
  const int32_t *cu_seqlens;
  // gate form (kGate*): general fp32 per-channel gates; pre-activations in
  // the input dtype (a, b, w and da, db, dw); coupled b = w = beta
  // ([.., T, H_v], db is then d(beta), dw unused); scalar, also a = alpha
  // ([.., T, H_v], da is then d(alpha))
  int gate_form;
};

// Kernel parameters: the arguments plus the three workspace regions (state
// checkpoints, per column block key-side partial sums, per-token k-reads).
struct BackwardParams {
  const void *q, *k, *v;
  const float *a, *b, *w, *S0;
  const void *dO;
  const float *dST;
  void *dq, *dk, *dv;
  float *da, *db, *dw, *dS0;
  float *ck, *part, *rk;
  float *wsum;
  const int32_t *cu;
  int B, T, H_qk, H_v, d_v;
  int gate_form;
};

size_t backward_workspace_bytes(int B, size_t BT, int H_v, int d_k, int d_v);
// The chunk-form backward (gdn2_backward_chunk.hip): whether it applies
// (unpacked bf16 sequences, d_k = d_v = 128, general gates, the prefill's
// 32-token chunk), its workspace, and the launch (*ran = false when some
// chunk decays too fast for it: nothing but the workspace written).
bool backward_chunked_eligible(const BackwardArgs &a);
size_t backward_chunked_workspace_bytes(int B, int T, int H_qk, int H_v);
hipError_t launch_backward_chunked(const BackwardArgs &a, hipStream_t st, bool *ran);
hipError_t launch_backward(const BackwardArgs &p, hipStream_t stream);
// Entering state of every segment of B sequences cut into nseg segments:
// S_in[(n * nseg + j) * H_v + h] = S0[n * H_v + h] (zero if S0 is null) for
// j = 0, else seg_states[j - 1] (PrefillArgs::seg_states); d_k x d_v fp32.
hipError_t launch_split_states(float *S_in, const float *S0, const float *seg_states, int B, int H_v, int nseg,
                               int dkdv, hipStream_t stream);
// Workspace of the backward of B sequences of T tokens: the split plan's
// when few long sequences run as segments, else backward_workspace_bytes.
size_t backward_workspace_bytes_split(int B, int T, int H_qk, int H_v, int d_k, int d_v, bool bf16);

hipError_t launch_decode(const DecodeArgs &p, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs &p, hipStream_t stream);
PrefillPlan prefill_plan(const PrefillArgs &p);
// Split-sequence hand-off: for j = 1 .. jlast in order,
// state[j] = trans[j] * state[j - 1] + state[j] per (sequence, head), where
// state is [nseg][BH][d_k][d_v] and trans [nseg][BH][d_k][d_k], fp32; then
// state[jlast] is also written to S_T ([BH][d_k][d_v]) if S_T is not null.
hipError_t launch_split_combine(float *state, const float *trans, int jlast, int BH, int d_k, int d_v,
                                float *S_T, hipStream_t stream);
// Output correction of split sequences (segments 1 .. nseg - 1 of B
// sequences of T tokens): o_t += oI_t . state[s - 1] per (sequence, value
// head), with oI [B*T][H_v][d_k] and o [B*T][H_v][d_v] in the input dtype.
hipError_t launch_split_correct(void *o, const void *oI, const float *state, int B, int T, int H_v, int d_k,
                                int d_v, int seg_len, int nseg, bool bf16, hipStream_t stream);
// Workgroup column width the prefill would use (for tests and tuning).
int prefill_pick_nct(int B, int H_v, int d_v);

}  // namespace gdn2
