/*
 * k3gen — seeded synthetic inputs for the routed MoE FFN layer.
 *
 * Input data only: this module holds none of the layer's arithmetic.  Both the
 * HIP path (through device buffers filled here or copied from host arrays made
 * here) and the CPU oracle (through host arrays made here) consume the bytes it
 * produces, so they see identical inputs.
 *
 * Random stream: a counter-based generator.  Draw i of stream `key` is the
 * SplitMix64 output function (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; constants as in Vigna's
 * reference splitmix64.c) applied to key + (i + 1) * 0x9E3779B97F4A7C15.
 * Any element of any tensor can therefore be regenerated on its own, on the
 * host or on the device, with integer arithmetic only.
 *
 * Element rules (identical on host and device):
 *   - packed E2M1 byte j of a tensor: byte (j mod 8) of draw j/8
 *     (little-endian), i.e. two uniformly random 4-bit codes;
 *   - E8M0 scale byte j: 127 + lo + floor(hi32(draw j) * (hi - lo + 1) / 2^32);
 *   - normal element j (host only): Box-Muller in fp64 on draws 2j and 2j+1,
 *     u1 = (d >> 11 + 1) * 2^-53, u2 = (d >> 11) * 2^-53,
 *     z = sqrt(-2 ln u1) * cos(2 pi u2), then sigma * z rounded to
 *     bf16 (round-to-nearest-even, in one step) or to fp32.
 */
#ifndef K3GEN_H
#define K3GEN_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Stream key of tensor `tensor_id` under `seed`. */
uint64_t k3gen_key(uint64_t seed, uint64_t tensor_id);
/* Draw i of stream `key`. */
uint64_t k3gen_draw(uint64_t key, uint64_t i);

/* Host fills; elements [start, start + n) of the tensor's stream. */
void k3gen_bytes(uint64_t key, uint64_t start, uint64_t n, uint8_t* out);
void k3gen_scales(uint64_t key, uint64_t start, uint64_t n, int lo, int hi, uint8_t* out);
void k3gen_normal_bf16(uint64_t key, uint64_t start, uint64_t n, double sigma, uint16_t* out);
void k3gen_normal_f32(uint64_t key, uint64_t start, uint64_t n, double sigma, float* out);

/* Device fills (libk3gen_dev.so); `out` is device memory, `stream` a
 * hipStream_t (NULL = default stream).  Return 0 on success, else the HIP
 * error code of the launch. */
int k3gen_dev_bytes(uint64_t key, uint64_t start, uint64_t n, uint8_t* out, void* stream);
int k3gen_dev_scales(uint64_t key, uint64_t start, uint64_t n, int lo, int hi, uint8_t* out,
                     void* stream);

#ifdef __cplusplus
}
#endif
#endif
