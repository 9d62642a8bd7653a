// Compile-time tile and occupancy knobs of the kernels: the fastest setting
// of each group in the sweep of attention_pass_cascaded_amd/tune.py on one
// MI355X (ms per call; every setting that was built and timed is listed).
// A -D on the compiler line overrides a value here.
#pragma once

// fwd:
//   RF_FWD_WAVES_D64=2: prefill causal 0.1465, prefill none 0.2490
//   RF_FWD_WAVES_D64=3: prefill causal 0.1430, prefill none 0.2437
//   RF_FWD_WAVES_D64=4: prefill causal 0.1425, prefill none 0.2436

// bwd:
//   RF_BWD_DQ_WAVES=2, RF_BWD_KV_WAVES=2, RF_BWD_BQ64=32: backward causal 0.4751
//   RF_BWD_DQ_WAVES=2, RF_BWD_KV_WAVES=2, RF_BWD_BQ64=64: backward causal 0.4314
//   RF_BWD_DQ_WAVES=2, RF_BWD_KV_WAVES=3, RF_BWD_BQ64=32: backward causal 0.4379
//   RF_BWD_DQ_WAVES=2, RF_BWD_KV_WAVES=3, RF_BWD_BQ64=64: backward causal 0.7448
//   RF_BWD_DQ_WAVES=3, RF_BWD_KV_WAVES=2, RF_BWD_BQ64=32: backward causal 0.4748
//   RF_BWD_DQ_WAVES=3, RF_BWD_KV_WAVES=2, RF_BWD_BQ64=64: backward causal 0.4338
//   RF_BWD_DQ_WAVES=3, RF_BWD_KV_WAVES=3, RF_BWD_BQ64=32: backward causal 0.4411
//   RF_BWD_DQ_WAVES=3, RF_BWD_KV_WAVES=3, RF_BWD_BQ64=64: backward causal 0.7468

#ifndef RF_FWD_WAVES_D64
#define RF_FWD_WAVES_D64 4
#endif
#ifndef RF_BWD_DQ_WAVES
#define RF_BWD_DQ_WAVES 2
#endif
#ifndef RF_BWD_KV_WAVES
#define RF_BWD_KV_WAVES 2
#endif
#ifndef RF_BWD_BQ64
#define RF_BWD_BQ64 64
#endif
