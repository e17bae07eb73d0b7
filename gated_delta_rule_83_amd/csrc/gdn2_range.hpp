// gdn2_range.hpp -- byte ranges of the prefill's raw buffer descriptors.
//
// A raw buffer descriptor carries a 32-bit byte range: accesses at or beyond
// it read 0 and writes are dropped, which is how the prefill handles ragged
// tails and requests issued past the last chunk without a branch. The range
// a chunk needs is never the rest of the sequence, only the tokens of that
// chunk, so it is computed from the chunk's window in 64 bits; the interface
// rejects problems whose window exceeds kMaxWindowBytes, so the result never
// wraps whatever the length of the sequence.
//
// Plain C++ (no HIP types) so that host code and host tests use the same
// function the kernels use.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define GDN2_HOST_DEVICE __host__ __device__
#else
#define GDN2_HOST_DEVICE
#endif

namespace gdn2 {

// Largest byte range one descriptor may need: a window of up to 64 tokens
// times the largest token stride of any tensor (the descriptor's range is a
// signed 32-bit quantity in the builtin that forms it).
constexpr uint64_t kMaxWindowBytes = 0x7fffffffull;
constexpr int kMaxWindowTokens = 64;

// Bytes from token t0 of a sequence of `len` tokens to the end of a window of
// at most `window` tokens, for a token stride of `stride` bytes; 0 at or past
// the end of the sequence. Exact for any len: the tokens left are counted in
// 64 bits and capped by the window before they are scaled.
GDN2_HOST_DEVICE inline uint32_t window_bytes(int64_t t0, int64_t len, int64_t window, uint32_t stride) {
  const int64_t left = len - t0;
  if (left <= 0 || window <= 0) return 0u;
  const uint64_t n = (uint64_t)(left < window ? left : window);
  const uint64_t bytes = n * (uint64_t)stride;
  return bytes > kMaxWindowBytes ? (uint32_t)kMaxWindowBytes : (uint32_t)bytes;
}

// Whether a prefill problem fits the descriptors: the largest token stride
// (bytes of one token row of any tensor: fp32 gates or state-dtype values)
// times the largest window. Problems beyond it are rejected at the interface.
GDN2_HOST_DEVICE inline bool window_fits(int64_t H_qk, int64_t H_v, int64_t d_k, int64_t d_v) {
  const int64_t h = H_qk > H_v ? H_qk : H_v;
  const int64_t d = d_k > d_v ? d_k : d_v;
  if (h <= 0 || d <= 0) return true;
  return (uint64_t)h * (uint64_t)d * 4u * (uint64_t)kMaxWindowTokens <= kMaxWindowBytes;
}

}  // namespace gdn2
