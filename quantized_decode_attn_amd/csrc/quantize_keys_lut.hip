// quantize_keys_lut.hip -- the codebook key-block kernels (see quantize_block.h for the steps).
#define KVQ_KEYS_LUT true
#define KVQ_KEYS_ENTRY launch_quantize_keys_lut
#include "quantize_keys.hip"
