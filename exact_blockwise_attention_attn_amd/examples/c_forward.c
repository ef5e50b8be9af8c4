/*
 * A C program that uses libattn through its C ABI alone: device buffers from
 * the HIP runtime, one causal forward (attn_fwd_partial) of seeded bf16
 * inputs, and the fp32 output O and the LSE written to a file.  No C++, no
 * Python, no torch.
 *
 * Usage: c_forward OUT_PATH
 * Output file: O [1, 300, 2, 128] fp32, then LSE [1, 2, 300] fp32.
 * Inputs: element i of tensor t (q = 0, k = 1, v = 2, [1, 300, 2, 128] each)
 * is example_value(t, i) below, a bf16 in [-1, 1).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "attn.h"

enum { B = 1, S = 300, H = 2, D = 128 };

/* A 32-bit integer hash of (tensor, index) mapped to [-1, 1) and cut to bf16. */
static uint16_t example_value(uint32_t t, uint32_t i) {
  uint32_t x = i * 2654435761u ^ (t + 1u) * 0x9E3779B9u;
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  const float f = (float)(x >> 8) / 8388608.0f - 1.0f;
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  return (uint16_t)(bits >> 16);
}

#define HIP_OK(call)                                                           \
  do {                                                                         \
    hipError_t e_ = (call);                                                    \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));      \
      return 1;                                                                \
    }                                                                          \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s OUT_PATH\n", argv[0]);
    return 2;
  }
  const size_t n = (size_t)B * S * H * D;
  uint16_t* h_in = (uint16_t*)malloc(n * sizeof(uint16_t));
  float* h_o = (float*)malloc(n * sizeof(float));
  float* h_lse = (float*)malloc((size_t)B * H * S * sizeof(float));
  if (!h_in || !h_o || !h_lse) return 1;

  void* d_in[3];
  for (uint32_t t = 0; t < 3; ++t) {
    for (size_t i = 0; i < n; ++i) h_in[i] = example_value(t, (uint32_t)i);
    HIP_OK(hipMalloc(&d_in[t], n * sizeof(uint16_t)));
    HIP_OK(hipMemcpy(d_in[t], h_in, n * sizeof(uint16_t), hipMemcpyHostToDevice));
  }
  void* d_o;
  void* d_lse;
  HIP_OK(hipMalloc(&d_o, n * sizeof(float)));
  HIP_OK(hipMalloc(&d_lse, (size_t)B * H * S * sizeof(float)));

  attn_fwd_args a;
  memset(&a, 0, sizeof a);
  a.struct_size = sizeof a;
  a.dtype = ATTN_DTYPE_BF16;
  a.batch = B;
  a.heads_q = H;
  a.heads_kv = H;
  a.seqlen_q = S;
  a.seqlen_k = S;
  a.head_dim = D;
  const int64_t st[3] = {(int64_t)S * H * D, (int64_t)H * D, D};
  a.q = d_in[0];
  a.k = d_in[1];
  a.v = d_in[2];
  memcpy(a.q_stride, st, sizeof st);
  memcpy(a.k_stride, st, sizeof st);
  memcpy(a.v_stride, st, sizeof st);
  a.o = d_o;
  memcpy(a.o_stride, st, sizeof st);
  a.o_dtype = ATTN_DTYPE_F32;
  a.lse = (float*)d_lse;
  a.causal = 1;
  a.flags = ATTN_FWD_BALANCED;

  const int status = attn_fwd_partial(&a, NULL);
  if (status != ATTN_OK) {
    fprintf(stderr, "attn_fwd_partial: %s: %s\n", attn_status_string(status), attn_last_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(h_o, d_o, n * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_lse, d_lse, (size_t)B * H * S * sizeof(float), hipMemcpyDeviceToHost));

  FILE* f = fopen(argv[1], "wb");
  if (!f) return 1;
  const int ok = fwrite(h_o, sizeof(float), n, f) == n &&
                 fwrite(h_lse, sizeof(float), (size_t)B * H * S, f) == (size_t)B * H * S;
  fclose(f);
  for (int t = 0; t < 3; ++t) HIP_OK(hipFree(d_in[t]));
  HIP_OK(hipFree(d_o));
  HIP_OK(hipFree(d_lse));
  free(h_in);
  free(h_o);
  free(h_lse);
  printf("attn_fwd_partial from C: ok (abi %d)\n", attn_abi_version());
  return ok ? 0 : 1;
}
