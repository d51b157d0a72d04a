// One-token decoder layers in one launch of resident workgroups
// (layer_resident.hip): shape, exchange area and launcher.
#pragma once

#include "common.hpp"

namespace w4a8 {
namespace resident {

// The layer shape the resident kernel serves: hidden 2048, feed-forward 8192
// (gate/up 2048 -> 16384, down 8192 -> 2048), qkv 2048 -> 2048 .. 4096.  One
// workgroup per 8 columns of o and down: 256 workgroups, all resident at once.
constexpr int kH = 2048;
constexpr int kF = 8192;
constexpr int kNbH = kH / kBlock;
constexpr int kNbF = kF / kBlock;
constexpr int kG = kH / 8;

// Exchange area (library-owned device memory, zeroed once): the epoch and
// error words on separate 128-byte lines, then the hand-over buffers of
// 64-bit words (32 bits of data, 32 bits of flag): the fp16 query slice (two
// columns per word), the residual stream after o, the quantised blocks of the
// gated product (eight words of codes and one scale per block), and the
// residual stream after down (the next layer's input inside one launch).
constexpr int kEpochWord = 0;
constexpr int kErrorWord = 64;
constexpr size_t kLlAOffset = 4096;
constexpr size_t kLlXOffset = kLlAOffset + size_t{kH / 2} * 8;
constexpr size_t kLlUOffset = kLlXOffset + size_t{kH} * 8;
constexpr size_t kLlYOffset = kLlUOffset + size_t{kNbF} * 9 * 8;
constexpr size_t kExchangeBytes = kLlYOffset + size_t{kH} * 8;

// Layers one launch runs (their weight pointers travel in the kernel
// arguments: 32 x 64 bytes).
constexpr int kMaxStack = 32;

struct LayerWeights {
  const uint8_t* qkv_w;
  const uint16_t* qkv_s;
  const uint8_t* o_w;
  const uint16_t* o_s;
  const uint8_t* gate_up_w;
  const uint16_t* gate_up_s;
  const uint8_t* down_w;
  const uint16_t* down_s;
};

struct StackArgs {
  float* x;  // fp32 [kH] residual stream, updated in place
  int n_qkv;
  int n_layers;  // 1 .. kMaxStack
  float alpha, eps;
  // The last layer's projection outputs, as the four-launch layer leaves them in its workspace.
  float* q;
  uint16_t* a;
  float* o;
  float* g;
  uint16_t* u;
  float* d;
  uint32_t* exchange;  // kExchangeBytes
  // Null: the layers start at qkv.  Otherwise one layer that starts at o, whose
  // fp16 [kH] input this is (the attention output between qkv and o); the
  // launch then runs no qkv phase and writes neither q nor a.
  const uint16_t* o_in;
  LayerWeights w[kMaxStack];
};

bool layer_supported(int H, int n_qkv, int n_gu);
// Workgroups of the resident kernel the device holds at once.
int co_resident_blocks(int* blocks);
int launch_stack(const StackArgs& a, hipStream_t stream);

}  // namespace resident
}  // namespace w4a8
