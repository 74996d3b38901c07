"""Single-GPU stand-ins for what surrounds the relayout path in a multi-GPU
Ulysses layer: the all-to-all exchange of P virtual ranks' wire buffers
(modelled as device copies inside one HBM) and the chunked schedule that
overlaps those exchanges with the relayout kernels.  Not part of the
library: on several GPUs an RCCL all-to-all takes the exchange's place."""
